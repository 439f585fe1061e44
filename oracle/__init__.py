"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in the package entry file and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports it and shares no code with
it; the only thing both sides consume is the seeded input generator, which
holds none of the method's arithmetic.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, OpenMP over the
independent (sequence, head) units).  This module is argument marshalling
through ctypes plus the build-on-demand of that C file.

Parity status: every function here is pinned by tests/test_oracle.py against
closed forms, invariants and a hand-worked example (see that file's header).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_L = ctypes.c_long


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = _build.LIB
    src = _build.SRC
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_gdn_recurrent.restype = ctypes.c_int
    lib.oracle_gdn_recurrent.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_void_p, _f64p, _f64p,
        _L, _L, _L, _L, ctypes.c_int, ctypes.c_int]
    lib.oracle_gdn_chunked.restype = ctypes.c_int
    lib.oracle_gdn_chunked.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_void_p, _f64p, _f64p,
        _L, _L, _L, _L, _L, ctypes.c_int]
    lib.oracle_gdn_chunk_stages.restype = ctypes.c_int
    lib.oracle_gdn_chunk_stages.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f64p, _L, _L] + [ctypes.c_void_p] * 8
    _LIB = lib
    return lib


def max_threads() -> int:
    """Threads the oracle's OpenMP runtime would use by default."""
    return int(_lib().oracle_max_threads())


def tile_key_heads(x, n_heads: int):
    """Expand q or k of n_key_heads heads to n_heads value heads in the tiled
    order: value head h takes key head h mod n_key_heads ("ggml attention
    kernels" model card, first bullet after the "Shapes, in torch order"
    table).  n_key_heads must divide n_heads."""
    x = np.asarray(x)
    hk = x.shape[2]
    if hk < 1 or n_heads % hk != 0:
        raise ValueError("n_key_heads must divide n_heads")
    return x[:, :, [h % hk for h in range(n_heads)]]


def _prep(q, k, v, g, beta, state):
    v = np.ascontiguousarray(v, dtype=np.float32)
    if np.ndim(q) == 4 and np.ndim(v) == 4 and np.shape(q)[2] != v.shape[2]:
        q = tile_key_heads(q, v.shape[2])
        k = tile_key_heads(k, v.shape[2])
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share shape (n_seqs, n_tokens, n_heads, d), or q "
                         "and k hold a divisor of n_heads key heads")
    S, T, H, d = q.shape
    if g.shape != (S, T, H) or beta.shape != (S, T, H):
        raise ValueError("g and beta must be (n_seqs, n_tokens, n_heads)")
    if state is not None:
        state = np.ascontiguousarray(state, dtype=np.float64)
        if state.shape != (S, H, d, d):
            raise ValueError("state must be (n_seqs, n_heads, d, d), [value][key]")
    return q, k, v, g, beta, state, (S, T, H, d)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# Input transforms the C oracle can apply first (see gdn_oracle.c)
L2NORM_QK = 1
RAW_GATES = 2


def gdn_recurrent(q, k, v, g, beta, state=None, threads: int = 0, l2norm_qk: bool = False,
                  raw_gates: bool = False):
    """Token-sequential fp64 recurrence.  Returns (out, final_state) as float64.

    q, k, v: (n_seqs, n_tokens, n_heads, d); g, beta: (n_seqs, n_tokens,
    n_heads); state: (n_seqs, n_heads, d, d) stored [value][key] or None for
    zeros.  q and k may hold fewer (key) heads, tiled over the value heads as
    ``tile_key_heads`` states.  Values are taken as given (bf16 inputs should
    be passed already rounded); all arithmetic is fp64.  ``l2norm_qk`` divides
    each q and k row by sqrt(|row|^2 + 1e-6) first; ``raw_gates`` takes g and
    beta as pre-activations, g <- -softplus(g) and beta <- sigmoid(beta).
    """
    q, k, v, g, beta, state, (S, T, H, d) = _prep(q, k, v, g, beta, state)
    out = np.empty((S, T, H, d), dtype=np.float64)
    fin = np.empty((S, H, d, d), dtype=np.float64)
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if raw_gates else 0)
    rc = _lib().oracle_gdn_recurrent(q, k, v, g, beta, _ptr(state), out, fin,
                                     S, T, H, d, flags, int(threads))
    if rc != 0:
        raise MemoryError("oracle_gdn_recurrent failed (%d)" % rc)
    return out, fin


def gdn_chunked(q, k, v, g, beta, state=None, chunk: int = 64, threads: int = 0):
    """The same result via the chunked (block) form, fp64.  Returns (out, final)."""
    q, k, v, g, beta, state, (S, T, H, d) = _prep(q, k, v, g, beta, state)
    out = np.empty((S, T, H, d), dtype=np.float64)
    fin = np.empty((S, H, d, d), dtype=np.float64)
    rc = _lib().oracle_gdn_chunked(q, k, v, g, beta, _ptr(state), out, fin,
                                   S, T, H, d, int(chunk), int(threads))
    if rc != 0:
        raise MemoryError("oracle_gdn_chunked failed (%d)" % rc)
    return out, fin


def chunk_stages(q, k, v, g, beta, state=None):
    """Stage values of ONE chunk for a single (seq, head).

    q, k, v: (n, d); g, beta: (n,); state: (d, d) [value][key] or None.
    Returns a dict with gam (n), A, T, P (n x n), W, U, Delta, out (n x d) and
    state (d x d, after the chunk).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    n, d = q.shape
    M = np.zeros((d, d)) if state is None else np.array(state, dtype=np.float64)
    M = np.ascontiguousarray(M)
    res = {"gam": np.empty(n), "A": np.empty((n, n)), "T": np.empty((n, n)),
           "P": np.empty((n, n)), "W": np.empty((n, d)), "U": np.empty((n, d)),
           "Delta": np.empty((n, d)), "out": np.empty((n, d))}
    rc = _lib().oracle_gdn_chunk_stages(
        q, np.ascontiguousarray(k, dtype=np.float32),
        np.ascontiguousarray(v, dtype=np.float32),
        np.ascontiguousarray(g, dtype=np.float32),
        np.ascontiguousarray(beta, dtype=np.float32), M, n, d,
        *[_ptr(res[key]) for key in ("gam", "A", "T", "P", "W", "U", "Delta", "out")])
    if rc != 0:
        raise MemoryError("oracle_gdn_chunk_stages failed (%d)" % rc)
    res["state"] = M
    return res


def chunk_lag_terms(k, g, beta, n, chunk: int = 64):
    """The two state-independent matrices through which chunk n's deltas depend on
    the deltas of the two chunks before it, for one (sequence, head).

    k: (n_tokens, d) keys; g, beta: (n_tokens,).  With gam the inclusive gate
    sums inside chunk n, c_m the total gate sum of chunk m, T_n = (I + A_n)^{-1}
    the chunk's triangular factor (``chunk_stages``) and K_m the key rows of chunk m:

        R1 = -T_n diag(beta e^gam) K_n K_{n-1}^T
        R2 = -e^{c_{n-1}} T_n diag(beta e^gam) K_n K_{n-2}^T

    (zero when the earlier chunk does not exist).  Then, with S_m the state
    entering chunk m and Dt_m = diag(e^{c_m - gam}) Delta_m,

        Delta_n = T_n E_n + R1 Dt_{n-1} + R2 Dt_{n-2},
        E_n = diag(beta)(V_n - e^{c_{n-1} + c_{n-2}} diag(e^gam) K_n S_{n-2}^T),

    which follows from writing S_n = e^{c_{n-1}} S_{n-1} + Dt_{n-1}^T K_{n-1} twice
    (the chunked form's state pass: Gated Delta Net on AMD, velstech.net, section
    "Why this bites AMD users specifically", the recurrence run in parallel blocks).
    Returns (R1, R2), each (rows of chunk n) x chunk, fp64."""
    k = np.asarray(k, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    beta = np.asarray(beta, dtype=np.float32)
    t0, t1 = n * chunk, min(len(g), (n + 1) * chunk)
    kn = k[t0:t1].astype(np.float64)
    st = chunk_stages(k[t0:t1], k[t0:t1], np.zeros_like(k[t0:t1]), g[t0:t1], beta[t0:t1])
    left = st["T"] @ np.diag(beta[t0:t1].astype(np.float64) * np.exp(st["gam"]))
    r1 = np.zeros((t1 - t0, chunk))
    r2 = np.zeros((t1 - t0, chunk))
    if n >= 1:
        kp = k[t0 - chunk:t0].astype(np.float64)
        r1 = -left @ kn @ kp.T
    if n >= 2:
        kpp = k[t0 - 2 * chunk:t0 - chunk].astype(np.float64)
        c_prev = np.sum(g[t0 - chunk:t0].astype(np.float64))
        r2 = -np.exp(c_prev) * (left @ kn @ kpp.T)
    return r1, r2


# ---- decode flash attention (the model card's second op, vector variant) -------

def flash_attn(q, k, v, mask=None, scale=None):
    """Softmax attention of a few queries over a key/value cache, fp64.

    Follows the "ggml attention kernels" model card, section "flash_attn":
    q (n_seqs, n_heads, n_q, d); k, v (n_seqs, n_heads_kv, n_kv, d) with query
    head h reading key/value head h // (n_heads / n_heads_kv) (grouped-query
    attention without an expanded copy; the card measures against repeat_kv,
    whose copies of key/value head j serve query heads j*g .. j*g + g - 1);
    mask (n_seqs, 1, n_q, n_kv) additive, cast to f16 first as the card says the
    kernel does, or None.  Returns (n_seqs, n_q, n_heads, d): tokens before
    heads.  scale defaults to 1 / sqrt(d).  A query row whose scores are all
    -inf (or an empty cache) gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, H, NQ, D = q.shape
    _, HKV, NKV, DV = v.shape
    if k.shape != (S, HKV, NKV, D) or v.shape[:3] != (S, HKV, NKV):
        raise ValueError("k, v must be (n_seqs, n_heads_kv, n_kv, d)")
    if HKV < 1 or H % HKV != 0:
        raise ValueError("n_heads_kv must divide n_heads")
    g = H // HKV
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    m16 = None
    if mask is not None:
        m16 = np.asarray(mask, dtype=np.float32).astype(np.float16).astype(np.float64)
        if m16.shape != (S, 1, NQ, NKV):
            raise ValueError("mask must be (n_seqs, 1, n_q, n_kv)")
    out = np.zeros((S, NQ, H, DV))
    for s in range(S):
        for h in range(H):
            j = h // g
            scores = sc * (q[s, h] @ k[s, j].T)               # (n_q, n_kv)
            if m16 is not None:
                scores = scores + m16[s, 0]
            for i in range(NQ):
                row = scores[i]
                top = np.max(row) if NKV else -np.inf
                if not np.isfinite(top):
                    continue                                  # nothing to attend to
                w = np.exp(row - top)
                out[s, i, h] = (w @ v[s, j]) / np.sum(w)
    return out
