"""libgdn Python binding: argument marshalling onto the C-ABI (include/gdn.h).

Every step of the gated delta rule runs in the HIP library; this module only
checks tensors, allocates outputs and the workspace with torch, and passes raw
device pointers and the current HIP stream through ctypes.  There is no CPU or
torch fallback: if the library cannot be loaded, calls raise.

Mirrors the op pair of the "ggml attention kernels" model card (section
"Ops"): ``forward(q, k, v, g, beta, state) -> (out, final_state)`` and
``supports(head_dim)``, with the shapes of its "Shapes, in torch order" table.
"""
import ctypes
import os

__all__ = ["forward", "prepare", "PreparedForward", "forward_noalloc", "noalloc_scratch_bytes",
           "supports", "workspace_size", "status_string", "library_path", "GdnError", "ALGOS",
           "flash_attn", "supports_flash_attn", "workspace_size_flash_attn"]

_PKG = os.path.dirname(os.path.abspath(__file__))
ALGOS = {"auto": 0, "recurrent": 1, "chunked": 2, "chunked_lag": 3, "chunked_head": 4}
# input transforms (gdn.h GDN_PRE_*)
PRE_L2NORM_QK = 1
PRE_RAW_GATES = 2
_DTYPES = {"f32": 0, "bf16": 1}
_LIB = None


class GdnError(RuntimeError):
    """A libgdn call returned a non-zero status."""

    def __init__(self, status, msg):
        super().__init__("libgdn status %d: %s" % (status, msg))
        self.status = status


def library_path() -> str:
    return os.environ.get("LIBGDN_PATH", os.path.join(_PKG, "libgdn.so"))


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("libgdn not built: %s is missing (run `python -m "
                           "linear_attention_recurrence_03_amd.build`)" % path)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.gdn_supports.restype = ctypes.c_int
    lib.gdn_supports.argtypes = [ctypes.c_int]
    lib.gdn_workspace_size.restype = ctypes.c_size_t
    lib.gdn_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.gdn_forward.restype = ctypes.c_int
    lib.gdn_forward.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                ctypes.c_int, vp, ctypes.c_size_t, ctypes.c_int, vp]
    lib.gdn_forward_tiled.restype = ctypes.c_int
    lib.gdn_forward_tiled.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                      i64, i64, ctypes.c_int, vp, ctypes.c_size_t,
                                      ctypes.c_int, vp]
    lib.gdn_forward_ex.restype = ctypes.c_int
    lib.gdn_forward_ex.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                   i64, i64, ctypes.c_int, ctypes.c_uint, vp, ctypes.c_size_t,
                                   ctypes.c_int, vp]
    lib.gdn_forward_noalloc.restype = ctypes.c_int
    lib.gdn_forward_noalloc.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                        i64, i64, ctypes.c_int, ctypes.c_uint, ctypes.c_int, vp]
    lib.gdn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.gdn_noalloc_scratch_bytes.argtypes = []
    lib.gdn_flash_attn_supports.restype = ctypes.c_int
    lib.gdn_flash_attn_supports.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.gdn_flash_attn_workspace_size.restype = ctypes.c_size_t
    lib.gdn_flash_attn_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.gdn_flash_attn.restype = ctypes.c_int
    lib.gdn_flash_attn.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                   ctypes.c_int, ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_version.restype = ctypes.c_int
    lib.gdn_version.argtypes = []
    _LIB = lib
    return lib


def supports(head_dim: int) -> bool:
    """True iff the library runs this head width (a multiple of 32, at most 128)."""
    return bool(_lib().gdn_supports(int(head_dim)))


def status_string(status: int) -> str:
    return _lib().gdn_status_string(int(status)).decode()


def workspace_size(dtype: str, n_seqs: int, n_tokens: int, n_heads: int, head_dim: int,
                   algo: str = "auto") -> int:
    """Device workspace bytes gdn_forward needs (0 for the token recurrence)."""
    return int(_lib().gdn_workspace_size(_DTYPES[dtype], n_seqs, n_tokens, n_heads, head_dim,
                                         ALGOS[algo]))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class PreparedForward:
    """One validated gdn_forward call with its C arguments built once.

    Calling it re-issues the same C call (the library validates again, in C) on
    the stream fixed at preparation, and returns ``(out, final_state)``.  It keeps
    the tensors it was prepared with alive; their contents may change between
    calls, their storage may not.  This is the cheap path for eager decode loops
    that call the op on the same buffers every step."""

    __slots__ = ("_fn", "_args", "_keep", "out", "state_out")

    def __init__(self, fn, args, keep, out, state_out):
        self._fn, self._args, self._keep = fn, args, keep
        self.out, self.state_out = out, state_out

    def __call__(self, stream=None):
        """Issue the call; ``stream`` (a torch stream) overrides the prepared one for
        this call only, e.g. to record it into a HIP graph being captured."""
        args = self._args
        if stream is not None:
            args = args[:-1] + (ctypes.c_void_p(stream.cuda_stream),)
        rc = self._fn(*args)
        if rc != 0:
            raise GdnError(rc, status_string(rc))
        return self.out, self.state_out


def prepare(q, k, v, g, beta, state=None, algo: str = "auto", out=None, state_out=None,
            workspace=None, stream=None, l2norm_qk: bool = False,
            raw_gates: bool = False) -> PreparedForward:
    """Validate the arguments of ``forward`` once, allocate what is missing and
    return a ``PreparedForward`` that issues the call.  Arguments are those of
    ``forward``.  Outputs and the workspace are allocated on ``stream`` (the
    caller's stream, else torch's current stream), the stream the call runs on,
    so torch's allocator never hands their memory to other work while the
    library may still use it."""
    import torch

    if q.dtype == torch.float32:
        dt = "f32"
    elif q.dtype == torch.bfloat16:
        dt = "bf16"
    else:
        raise TypeError("q/k/v must be float32 or bfloat16, got %s" % q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype %s differs from q dtype %s" % (name, t.dtype, q.dtype))
    if q.dim() != 4 or v.dim() != 4 or k.shape != q.shape or \
            q.shape[:2] != v.shape[:2] or q.shape[3] != v.shape[3]:
        raise ValueError("q, k must be (n_seqs, n_tokens, n_key_heads, head_dim) and v "
                         "(n_seqs, n_tokens, n_heads, head_dim)")
    S, T, H, D = v.shape
    HK = q.shape[2]
    if g.shape != (S, T, H) or beta.shape != (S, T, H):
        raise ValueError("g and beta must be (n_seqs, n_tokens, n_heads)")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    if state is not None:
        if state.shape != (S, H, D, D) or state.dtype != torch.float32:
            raise ValueError("state must be float32 (n_seqs, n_heads, d, d)")
    tensors = [q, k, v, g, beta] + ([state] if state is not None else [])
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    dev = q.device
    if out is not None and (out.shape != v.shape or out.dtype != v.dtype or not out.is_cuda
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like v")
    if state_out is not None and (state_out.shape != (S, H, D, D) or not state_out.is_cuda
                                  or state_out.dtype != torch.float32
                                  or not state_out.is_contiguous()):
        raise ValueError("state_out must be a contiguous float32 (n_seqs, n_heads, d, d) "
                         "GPU tensor")
    a = ALGOS[algo]
    lib = _lib()
    need = int(lib.gdn_workspace_size(_DTYPES[dt], S, T, H, D, a))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.stream(stream):   # allocations belong to the stream that uses them
        if out is None:
            out = torch.empty_like(v)
        if state_out is None:
            state_out = torch.empty((S, H, D, D), dtype=torch.float32, device=dev)
        if need > 0 and (workspace is None or
                         workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    handle = ctypes.c_void_p(stream.cuda_stream)
    flags = (PRE_L2NORM_QK if l2norm_qk else 0) | (PRE_RAW_GATES if raw_gates else 0)
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
            _ptr(state_out))
    tail = (_ptr(workspace), ctypes.c_size_t(ws_bytes), ctypes.c_int(a), handle)
    i64 = ctypes.c_int64
    if flags:
        fn = lib.gdn_forward_ex
        args = (_DTYPES[dt],) + ptrs + (i64(S), i64(T), i64(H), i64(HK), ctypes.c_int(D),
                                        ctypes.c_uint(flags)) + tail
    elif HK == H:
        fn = lib.gdn_forward
        args = (_DTYPES[dt],) + ptrs + (i64(S), i64(T), i64(H), ctypes.c_int(D)) + tail
    else:
        fn = lib.gdn_forward_tiled
        args = (_DTYPES[dt],) + ptrs + (i64(S), i64(T), i64(H), i64(HK),
                                        ctypes.c_int(D)) + tail
    keep = (q, k, v, g, beta, state, workspace, stream)
    return PreparedForward(fn, args, keep, out, state_out)


def forward(q, k, v, g, beta, state=None, algo: str = "auto", out=None, state_out=None,
            workspace=None, stream=None, l2norm_qk: bool = False, raw_gates: bool = False):
    """Run the gated delta rule over all tokens.  Returns (out, final_state).

    q, k, v: (n_seqs, n_tokens, n_heads, head_dim) float32 or bfloat16 CUDA
    tensors (same dtype).  q and k may instead hold n_key_heads heads, a
    divisor of n_heads: value head h then reads key/query head h % n_key_heads
    (the tiled order; ``gdn_forward_tiled``).  g, beta: (n_seqs, n_tokens,
    n_heads) float32; state:
    (n_seqs, n_heads, head_dim, head_dim) float32 stored [value][key], or None
    for zeros.  ``state_out`` may be ``state`` itself for an in-place update.
    ``l2norm_qk`` normalises each q and k row inside the op; ``raw_gates`` takes
    g and beta as pre-activations (g := -softplus(g), beta := sigmoid(beta)).
    Work is enqueued on ``stream`` (default: torch's current stream), where the
    outputs and the workspace are also allocated; nothing is synchronised.
    """
    return prepare(q, k, v, g, beta, state, algo=algo, out=out, state_out=state_out,
                   workspace=workspace, stream=stream, l2norm_qk=l2norm_qk,
                   raw_gates=raw_gates)()


def forward_noalloc(q, k, v, g, beta, state, out, state_out, algo: str = "auto", stream=None,
                    l2norm_qk: bool = False, raw_gates: bool = False):
    """``forward`` through gdn_forward_noalloc: no workspace and no allocation, the
    chunked algorithm's scratch being the library's fixed per-GPU array
    (``noalloc_scratch_bytes()``).  ``out`` and ``state_out`` must be given (shaped
    as in ``forward``); the arguments are passed to the C call as they are and the
    library validates them.  Returns (out, state_out)."""
    import torch
    dt = "bf16" if q.dtype == torch.bfloat16 else "f32"
    S, T, H, D = v.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    flags = (PRE_L2NORM_QK if l2norm_qk else 0) | (PRE_RAW_GATES if raw_gates else 0)
    rc = _lib().gdn_forward_noalloc(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state), _ptr(out), _ptr(state_out), S, T, H,
                                    q.shape[2], D, flags, ALGOS[algo],
                                    ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise GdnError(rc, status_string(rc))
    return out, state_out


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-GPU scratch array behind gdn_forward_noalloc."""
    return int(_lib().gdn_noalloc_scratch_bytes())


def supports_flash_attn(n_q: int, head_dim_k: int, head_dim_v: int) -> bool:
    """True iff the decode attention runs these sizes (1 <= n_q < 20, equal key and
    value widths of 64, 128 or 256)."""
    return bool(_lib().gdn_flash_attn_supports(int(n_q), int(head_dim_k), int(head_dim_v)))


def workspace_size_flash_attn(n_seqs: int, n_heads: int, n_heads_kv: int, n_q: int,
                              n_kv: int, head_dim: int) -> int:
    """Device workspace bytes gdn_flash_attn needs for these sizes (0: none)."""
    return int(_lib().gdn_flash_attn_workspace_size(n_seqs, n_heads, n_heads_kv, n_q, n_kv,
                                                    head_dim))


def flash_attn(q, k, v, mask=None, scale=None, out=None, workspace=None, stream=None):
    """Decode attention of a few queries over a key/value cache ("ggml attention
    kernels" model card, section "flash_attn").  Returns out.

    q: (n_seqs, n_heads, n_q, d); k, v: (n_seqs, n_heads_kv, n_kv, d), float32 or
    bfloat16 CUDA tensors of one dtype, n_heads_kv dividing n_heads (query head h
    reads key/value head h // (n_heads / n_heads_kv)); mask: (n_seqs, 1, n_q,
    n_kv) additive (converted to float32 here; the op rounds it to f16) or None;
    scale defaults to 1/sqrt(d).  out: (n_seqs, n_q, n_heads, d), like q.
    """
    import torch
    if q.dtype == torch.float32:
        dt = "f32"
    elif q.dtype == torch.bfloat16:
        dt = "bf16"
    else:
        raise TypeError("q/k/v must be float32 or bfloat16, got %s" % q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype %s differs from q dtype %s" % (name, t.dtype, q.dtype))
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or \
            k.shape[3] != q.shape[3]:
        raise ValueError("q must be (n_seqs, n_heads, n_q, d) and k, v (n_seqs, n_heads_kv, "
                         "n_kv, d)")
    S, H, NQ, D = q.shape
    HKV, NKV = k.shape[1], k.shape[2]
    if mask is not None and mask.shape != (S, 1, NQ, NKV):
        raise ValueError("mask must be (n_seqs, 1, n_q, n_kv)")
    if out is not None and (out.shape != (S, NQ, H, D) or out.dtype != q.dtype
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous (n_seqs, n_q, n_heads, d) tensor like q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    lib = _lib()
    need = int(lib.gdn_flash_attn_workspace_size(S, H, HKV, NQ, NKV, D))
    # the converted mask, the output and the workspace belong to the stream that uses them
    with torch.cuda.stream(stream):
        if mask is not None:
            mask = mask.to(torch.float32).contiguous()
        if out is None:
            out = torch.empty((S, NQ, H, D), dtype=q.dtype, device=q.device)
        if need > 0 and (workspace is None or
                         workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    for t in (q, k, v, out) + ((mask,) if mask is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.gdn_flash_attn(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(out),
                            S, H, HKV, NQ, NKV, D, sc, _ptr(workspace), ws_bytes,
                            ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise GdnError(rc, status_string(rc))
    return out
