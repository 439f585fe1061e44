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

__all__ = ["forward", "supports", "workspace_size", "status_string", "library_path",
           "GdnError", "ALGOS", "flash_attn", "supports_flash_attn",
           "workspace_size_flash_attn"]

_PKG = os.path.dirname(os.path.abspath(__file__))
ALGOS = {"auto": 0, "recurrent": 1, "chunked": 2}
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
    Work is enqueued on ``stream`` (default: torch's current stream); nothing
    is synchronised.
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
    if out is None:
        out = torch.empty_like(v)
    if state_out is None:
        state_out = torch.empty((S, H, D, D), dtype=torch.float32, device=dev)
    a = ALGOS[algo]
    lib = _lib()
    need = int(lib.gdn_workspace_size(_DTYPES[dt], S, T, H, D, a))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(stream.cuda_stream)
    flags = (PRE_L2NORM_QK if l2norm_qk else 0) | (PRE_RAW_GATES if raw_gates else 0)
    if flags:
        rc = lib.gdn_forward_ex(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(state), _ptr(out), _ptr(state_out), S, T, H, HK, D, flags,
                                _ptr(workspace), ws_bytes, a, handle)
    elif HK == H:
        rc = lib.gdn_forward(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state), _ptr(out), _ptr(state_out), S, T, H, D,
                             _ptr(workspace), ws_bytes, a, handle)
    else:
        rc = lib.gdn_forward_tiled(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out), S, T,
                                   H, HK, D, _ptr(workspace), ws_bytes, a, handle)
    if rc != 0:
        raise GdnError(rc, status_string(rc))
    return out, state_out


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
    if mask is not None:
        if mask.shape != (S, 1, NQ, NKV):
            raise ValueError("mask must be (n_seqs, 1, n_q, n_kv)")
        mask = mask.to(torch.float32).contiguous()
    for t in (q, k, v) + ((mask,) if mask is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    if out is None:
        out = torch.empty((S, NQ, H, D), dtype=q.dtype, device=q.device)
    elif out.shape != (S, NQ, H, D) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (n_seqs, n_q, n_heads, d) tensor like q")
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    lib = _lib()
    need = int(lib.gdn_flash_attn_workspace_size(S, H, HKV, NQ, NKV, D))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = lib.gdn_flash_attn(_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(out),
                            S, H, HKV, NQ, NKV, D, sc, _ptr(workspace), ws_bytes,
                            ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise GdnError(rc, status_string(rc))
    return out
