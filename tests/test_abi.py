"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, answers gdn_supports / gdn_workspace_size / gdn_status_string,
and rejects bad arguments on the host before any launch.

Only error paths and no-op calls are made here; all of them return before the
library touches the HIP runtime.  Pointers are fake, aligned integers.
"""
import ctypes
import os
import re

import pytest

import linear_attention_recurrence_03_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

F32, BF16 = 0, 1
AUTO, REC, CHUNK = 0, 1, 2
OK, E_HD, E_SHAPE, E_NULL, E_DTYPE, E_WS, E_ALGO, E_ALIGN, E_ALIAS, E_HIP = \
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def lib():
    path = gdn.library_path()
    if not os.path.exists(path):
        pytest.fail("libgdn.so is not built; run python -m linear_attention_recurrence_03_amd.build")
    return gdn._lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _declared_functions()
    assert {"gdn_forward", "gdn_supports", "gdn_workspace_size", "gdn_status_string",
            "gdn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "symbol %s declared in gdn.h but not exported" % n


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    codes = dict((m.group(1), int(m.group(2)))
                 for m in re.finditer(r"(GDN_(?:OK|ERR_[A-Z_]+))\s*=\s*(-?\d+)", text))
    assert codes["GDN_OK"] == OK and codes["GDN_ERR_HIP"] == E_HIP
    assert codes["GDN_ERR_ALIASING"] == E_ALIAS and codes["GDN_ERR_MISALIGNED"] == E_ALIGN


def test_supports_truth_table(lib):
    yes = {32, 64, 96, 128}
    for d in range(-1, 300):
        assert lib.gdn_supports(d) == (1 if d in yes else 0), d
    assert gdn.supports(128) and not gdn.supports(256) and not gdn.supports(48)


def test_status_strings(lib):
    for s in range(-12, 2):
        txt = gdn.status_string(s)
        assert isinstance(txt, str) and txt
    assert gdn.status_string(0) == "ok"
    assert "head_dim" in gdn.status_string(E_HD)
    assert lib.gdn_version() >= 100


def test_workspace_size(lib):
    assert gdn.workspace_size("f32", 1, 1, 32, 128, "auto") == 0       # recurrence
    # AUTO's crossover (first chunked token count) by work w = seqs * heads * (d/128)^2
    for dtype, n_seqs, n_heads, d, first in (
            ("bf16", 1, 32, 128, 20), ("bf16", 2, 32, 128, 20), ("bf16", 4, 32, 128, 18),
            ("bf16", 8, 32, 128, 16), ("bf16", 32, 32, 128, 14),
            ("bf16", 1, 128, 64, 20),                                  # w = 32
            ("f32", 1, 32, 128, 48), ("f32", 2, 32, 128, 60), ("f32", 4, 32, 128, 104),
            ("f32", 64, 32, 128, 120)):
        assert gdn.workspace_size(dtype, n_seqs, first - 1, n_heads, d, "auto") == 0
        assert gdn.workspace_size(dtype, n_seqs, first, n_heads, d, "auto") > 0
    assert gdn.workspace_size("bf16", 1, 4096, 32, 128, "recurrent") == 0
    assert gdn.workspace_size("bf16", 0, 4096, 32, 128, "chunked") == 0
    assert gdn.workspace_size("bf16", 1, 4096, 32, 48, "chunked") == 0  # unsupported
    big = gdn.workspace_size("bf16", 1, 4096, 32, 128, "chunked")
    small = gdn.workspace_size("bf16", 1, 64, 32, 128, "chunked")
    assert big >= small >= 0
    assert lib.gdn_workspace_size(7, 1, 64, 1, 32, 0) == 0               # bad dtype
    assert lib.gdn_workspace_size(0, 1, 64, 1, 32, 9) == 0               # bad algo
    # the two-chunk-lag form: bf16 only, 30 KiB per (seq, head, chunk) against 14 KiB
    assert gdn.workspace_size("f32", 1, 4096, 32, 128, "chunked_lag") == 0
    lag = gdn.workspace_size("bf16", 1, 4096, 32, 128, "chunked_lag")
    assert lag == 32 * 64 * 30 * 1024 and big == 32 * 64 * 14 * 1024
    assert gdn.workspace_size("bf16", 1, 4096 + 1, 32, 128, "chunked_lag") == 32 * 65 * 30 * 1024
    # the whole-head pass reads the same workspace as the per-tile one
    assert gdn.workspace_size("bf16", 1, 4096, 32, 128, "chunked_head") == big
    assert gdn.workspace_size("f32", 1, 4096, 32, 128, "chunked_head") == 0


class _Call:
    """Builds gdn_forward arguments with fake, non-overlapping aligned pointers."""

    def __init__(self, S=1, T=4, H=2, D=32, dtype=F32):
        self.S, self.T, self.H, self.D, self.dtype = S, T, H, D, dtype
        esz = 2 if dtype == BF16 else 4
        tok = max(S * T * H * D * esz, 16)
        gate = max(S * T * H * 4, 16)
        st = max(S * H * D * D * 4, 16)
        base = 1 << 32
        sizes = [("q", tok), ("k", tok), ("v", tok), ("g", gate), ("beta", gate),
                 ("state_in", st), ("out", tok), ("state_out", st), ("ws", 1 << 30)]
        self.p = {}
        for name, size in sizes:
            self.p[name] = base
            base += (size + 4095) // 4096 * 4096 + 4096
        self.ws_bytes = 0
        self.algo = REC

    def __call__(self, lib, **over):
        a = dict(self.p)
        a.update(over)
        S, T, H, D = (over.pop(x, getattr(self, x)) for x in ("S", "T", "H", "D"))
        return lib.gdn_forward(over.get("dtype", self.dtype), a["q"], a["k"], a["v"], a["g"],
                               a["beta"], a["state_in"], a["out"], a["state_out"], S, T, H,
                               over.get("D", D), a["ws"], over.get("ws_bytes", self.ws_bytes),
                               over.get("algo", self.algo), None)


def test_forward_rejects_before_launch(lib):
    c = _Call()
    assert c(lib, D=48) == E_HD
    assert c(lib, D=256) == E_HD
    assert c(lib, dtype=5) == E_DTYPE
    assert c(lib, algo=3) == E_ALGO          # the lag form has no fp32 variant
    assert c(lib, algo=4) == E_ALGO          # nor the whole-head pass
    assert c(lib, algo=5) == E_ALGO
    assert c(lib, algo=4, dtype=BF16) == E_WS
    assert c(lib, algo=3, dtype=BF16) == E_WS  # bf16: accepted, needs its workspace
    assert c(lib, S=-1) == E_SHAPE
    assert c(lib, T=-2) == E_SHAPE
    assert c(lib, H=1 << 62) == E_SHAPE
    assert c(lib, q=None) == E_NULL
    assert c(lib, beta=None) == E_NULL
    assert c(lib, out=None) == E_NULL
    assert c(lib, state_out=None) == E_NULL
    assert c(lib, k=c.p["k"] + 4) == E_ALIGN
    assert c(lib, state_in=c.p["state_in"] + 8) == E_ALIGN
    # out overlapping an input, state_out overlapping an input or partially state_in
    assert c(lib, out=c.p["q"]) == E_ALIAS
    assert c(lib, out=c.p["state_out"]) == E_ALIAS
    assert c(lib, state_out=c.p["g"]) == E_ALIAS
    assert c(lib, state_out=c.p["state_in"] + 16) == E_ALIAS
    assert c(lib, out=c.p["state_in"]) == E_ALIAS


def test_forward_chunked_workspace_checks(lib):
    c = _Call(T=130, H=2, D=64, dtype=BF16)
    need = lib.gdn_workspace_size(BF16, 1, 130, 2, 64, CHUNK)
    if need == 0:
        pytest.skip("chunked path needs no workspace")
    assert c(lib, algo=CHUNK, ws_bytes=need - 1) == E_WS
    assert c(lib, algo=CHUNK, ws_bytes=need, ws=None) == E_NULL
    assert c(lib, algo=CHUNK, ws_bytes=need, ws=c.p["q"]) == E_ALIAS


def test_forward_noops_without_gpu(lib):
    c = _Call()
    # n_seqs == 0 or n_heads == 0: nothing to do, even with null pointers
    assert c(lib, S=0, q=None, k=None, v=None, g=None, beta=None, out=None,
             state_out=None) == OK
    assert c(lib, H=0) == OK
    # n_tokens == 0 with state_out == state_in: nothing to launch
    assert c(lib, T=0, q=None, k=None, v=None, g=None, beta=None, out=None,
             state_out=c.p["state_in"]) == OK


def _tiled(lib, c, HK, **over):
    """gdn_forward_tiled with the pointers of _Call c (q, k sized for H heads, so
    any HK <= H fits).  Every call here must fail validation or be a no-op."""
    a = dict(c.p)
    a.update(over)
    return lib.gdn_forward_tiled(c.dtype, a["q"], a["k"], a["v"], a["g"], a["beta"],
                                 a["state_in"], a["out"], a["state_out"], over.get("S", c.S),
                                 over.get("T", c.T), over.get("H", c.H), HK, c.D, a["ws"],
                                 over.get("ws_bytes", c.ws_bytes), over.get("algo", c.algo),
                                 None)


def test_forward_tiled_rejects_before_launch(lib):
    c = _Call(H=6)
    assert _tiled(lib, c, 0) == E_SHAPE          # no key heads
    assert _tiled(lib, c, -2) == E_SHAPE
    assert _tiled(lib, c, 4) == E_SHAPE          # 4 does not divide 6
    assert _tiled(lib, c, 7) == E_SHAPE          # more key heads than value heads
    assert _tiled(lib, c, 3, q=None) == E_NULL
    assert _tiled(lib, c, 3, k=c.p["k"] + 4) == E_ALIGN
    assert _tiled(lib, c, 3, out=c.p["q"]) == E_ALIAS
    assert _tiled(lib, c, 2, state_out=c.p["k"]) == E_ALIAS
    # n_heads == 0 is a no-op whatever the (non-negative) key-head count
    assert _tiled(lib, c, 0, H=0) == OK
    assert _tiled(lib, c, 5, S=0) == E_SHAPE     # not a divisor of 6, even with no sequences
    assert _tiled(lib, c, -1, H=0) == E_SHAPE


def test_forward_tiled_q_extent_uses_key_heads(lib):
    """q and k span n_key_heads heads: an output placed right after a one-head q
    passes the aliasing checks (the call then stops at the workspace check, the
    last one before a launch), one that starts inside it does not."""
    c = _Call(H=4, T=64, D=32)
    one_head_q = 1 * 64 * 1 * 32 * 4
    q = c.p["ws"]  # q in the free region, so that only q can meet out
    chunked = dict(algo=CHUNK, ws_bytes=0, q=q)
    assert _tiled(lib, c, 1, out=q + one_head_q, **chunked) == E_WS
    assert _tiled(lib, c, 1, out=q + one_head_q - 16, **chunked) == E_ALIAS
    assert _tiled(lib, c, 4, out=q + one_head_q, **chunked) == E_ALIAS


def test_forward_ex_flags(lib):
    """gdn_forward_ex: unknown transform bits are rejected; known ones pass the
    flag check and the call stops at the next failing check (no launch)."""
    c = _Call(H=4)
    a = c.p

    def ex(flags, HK=4, **over):
        b = dict(a)
        b.update(over)
        return lib.gdn_forward_ex(c.dtype, b["q"], b["k"], b["v"], b["g"], b["beta"],
                                  b["state_in"], b["out"], b["state_out"], c.S, c.T, c.H, HK,
                                  c.D, flags, b["ws"], 0, c.algo, None)
    E_FLAGS = -10
    for bad in (4, 8, 1 << 31, 0xFFFFFFFF):
        assert ex(bad) == E_FLAGS
    for ok in (0, 1, 2, 3):
        assert ex(ok, q=None) == E_NULL
        assert ex(ok, out=a["q"]) == E_ALIAS
        assert ex(ok, HK=3) == E_SHAPE
    assert "flag" in gdn.status_string(E_FLAGS)


def test_flash_attn_host_checks(lib):
    """Decode attention: supports table, workspace query and rejections before any
    launch (fake pointers; every call fails validation or is a no-op)."""
    assert lib.gdn_flash_attn_supports(1, 256, 256) == 1
    assert lib.gdn_flash_attn_supports(19, 64, 64) == 1
    assert lib.gdn_flash_attn_supports(20, 64, 64) == 0
    assert lib.gdn_flash_attn_supports(0, 64, 64) == 0
    assert lib.gdn_flash_attn_supports(1, 128, 64) == 0
    assert lib.gdn_flash_attn_supports(1, 96, 96) == 0
    assert lib.gdn_flash_attn_workspace_size(1, 16, 4, 1, 512, 256) > 0
    assert lib.gdn_flash_attn_workspace_size(1, 16, 3, 1, 512, 256) == 0   # bad ratio
    assert lib.gdn_flash_attn_workspace_size(1, 16, 4, 1, 512, 96) == 0    # bad width
    base = 1 << 32
    q, k, v, m, o = (base + i * (1 << 24) for i in range(5))
    ws = base + 6 * (1 << 24)

    def fa(dtype=F32, q=q, k=k, v=v, m=m, o=o, S=1, H=4, HKV=2, NQ=2, NKV=100, D=64,
           scale=0.125, ws=ws, ws_bytes=0):
        return lib.gdn_flash_attn(dtype, q, k, v, m, o, S, H, HKV, NQ, NKV, D,
                                  ctypes.c_float(scale), ws, ws_bytes, None)
    assert fa(D=96) == E_HD
    assert fa(dtype=3) == E_DTYPE
    assert fa(NQ=20) == E_SHAPE
    assert fa(NQ=0) == E_SHAPE
    assert fa(HKV=3) == E_SHAPE
    assert fa(NKV=-1) == E_SHAPE
    assert fa(scale=float("nan")) == E_SHAPE
    assert fa(q=None) == E_NULL
    assert fa(k=None) == E_NULL
    assert fa(q=q + 4) == E_ALIGN
    assert fa(o=q) == E_ALIAS
    assert fa(o=m + 16) == E_ALIAS
    need = lib.gdn_flash_attn_workspace_size(1, 4, 2, 2, 100, 64)
    if need > 0:
        assert fa(ws_bytes=need - 1) == E_WS
        assert fa(ws_bytes=need, ws=None) == E_NULL
    assert fa(S=0, q=None, k=None, v=None, m=None, o=None) == OK
    assert fa(H=0, HKV=0) == OK


def test_size_limits(lib):
    """Calls whose grids would not fit one dispatch (work-items counted in 32 bits)
    are rejected up front: at most 2^27 state rows, fewer than 2^24 chunks for the
    chunked form, and decode-attention grids that fit.  Accepted shapes reach the
    pointer checks (null q: GDN_ERR_NULL_POINTER), so nothing is launched either way."""
    rows = 1 << 27
    c = _Call(T=1, H=1, D=128)
    assert c(lib, S=rows // 128, q=None) == E_NULL
    assert c(lib, S=rows // 128 + 1, q=None) == E_SHAPE
    c32 = _Call(T=1, H=4, D=32)
    assert c32(lib, S=rows // 128, q=None) == E_NULL
    assert c32(lib, S=rows // 128 + 1, q=None) == E_SHAPE
    # chunks: n_seqs * n_heads * ceil(n_tokens / 64) < 2^24 when the chunked form runs
    nmax = (1 << 24) - 1
    assert gdn.workspace_size("bf16", 1, nmax * 64, 1, 32, "chunked") > 0
    assert gdn.workspace_size("bf16", 1, nmax * 64 + 1, 1, 32, "chunked") == 0
    assert gdn.workspace_size("bf16", 2, (nmax // 2) * 64, 1, 32, "auto") > 0
    assert gdn.workspace_size("bf16", 2, (nmax // 2 + 1) * 64, 1, 32, "auto") == 0
    cl = _Call(S=1, H=1, D=32, dtype=BF16)
    assert cl(lib, T=nmax * 64 + 1, algo=CHUNK, q=None) == E_SHAPE
    assert cl(lib, T=nmax * 64 + 1, algo=REC, q=None) == E_NULL   # the recurrence has no chunks
    # decode attention: 2^24 single-row (seq, head) units of 256 work-items overflow
    base = 1 << 32

    def fa(S, H=1, HKV=1, NQ=1, NKV=64, q=base):
        return lib.gdn_flash_attn(F32, q, base + (1 << 40), base + (2 << 40), None,
                                  base + (3 << 40), S, H, HKV, NQ, NKV, 64,
                                  ctypes.c_float(0.125), None, 0, None)
    assert fa(S=(1 << 24) - 1, q=None) == E_NULL
    assert fa(S=1 << 24, q=None) == E_SHAPE
    assert fa(S=1 << 22, H=4, HKV=1, NQ=1, q=None) == E_NULL     # four rows per workgroup
    assert fa(S=(1 << 24) + 1, q=None) == E_SHAPE
    # cache positions are indexed in 32 bits: fewer than 2^31
    assert fa(S=1, NKV=(1 << 31) - 1, q=None) == E_NULL
    assert fa(S=1, NKV=1 << 31, q=None) == E_SHAPE


def test_chunk_row_span_limit(lib):
    """The chunked kernels address a token row inside one 64-token chunk with a
    32-bit byte offset, so a chunked call whose 64 rows of all heads reach 4 GiB
    (64 * n_heads * head_dim * element size >= 2^32) is rejected; the token
    recurrence has no such limit."""
    for dtype, esz in ((BF16, 2), (F32, 4)):
        hmax = (1 << 32) // (64 * 128 * esz) - 1        # 262143 (bf16), 131071 (fp32)
        c = _Call(S=1, T=64, D=128, dtype=dtype)
        assert c(lib, H=hmax, algo=CHUNK, q=None) == E_NULL
        assert c(lib, H=hmax + 1, algo=CHUNK, q=None) == E_SHAPE
        assert c(lib, H=hmax + 1, algo=REC, q=None) == E_NULL
        name = "bf16" if dtype == BF16 else "f32"
        assert gdn.workspace_size(name, 1, 64, hmax, 128, "chunked") > 0
        assert gdn.workspace_size(name, 1, 64, hmax + 1, 128, "chunked") == 0


def test_noalloc_refuses_beyond_scratch_before_launch(lib):
    """gdn_forward_noalloc checks the chunked workspace it would need against its
    fixed scratch array first: a larger call returns GDN_ERR_SCRATCH_TOO_SMALL with
    no HIP call (so this runs without a GPU); a fitting call reaches the pointer
    checks of gdn_forward_ex."""
    E_SCRATCH = -11
    cap = lib.gdn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    base = 1 << 32

    def call(S, T, H, q=base):
        return lib.gdn_forward_noalloc(BF16, q, base + (1 << 40), base + (2 << 40),
                                       base + (3 << 40), base + (4 << 40), None,
                                       base + (5 << 40), base + (6 << 40), S, T, H, H, 128, 0,
                                       CHUNK, None)
    per_seq = lib.gdn_workspace_size(BF16, 1, 4096, 32, 128, CHUNK)
    fits = cap // per_seq
    assert fits >= 1
    assert call(fits, 4096, 32, q=None) == E_NULL
    assert call(fits + 1, 4096, 32) == E_SCRATCH
    assert "scratch" in lib.gdn_status_string(E_SCRATCH).decode()
    assert call(1, 4096, 32, q=None) == E_NULL
