"""Python binding of libfa (include/fa.h): exact IO-aware attention on MI355X.

Argument marshalling only.  Every step of the attention path runs in the HIP
kernels of libfa.so; PyTorch is used to allocate device memory and to supply
the stream.  There is no fallback: if the library is missing, importing the
binding's functions raises.

Low-level functions carry the C names and take caller-allocated tensors:
    fa_fwd(q, k, v, o, lse, scale, causal)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal)
    fa_decode(q, k, v, o, lse, scale, num_splits, workspace)
    fa_decode_varlen(q, k, v, kv_lens, o, lse, scale, num_splits, workspace): decode
        over a padded cache of ragged per-sequence histories
    fa_decode_noalloc(q, k, v, o, lse, scale, num_splits): fa_decode_ex without a
        workspace argument (the library's static device scratch instead), for
        callers that cannot allocate
    fa_fwd_ex / fa_bwd_ex / fa_decode_ex: the same with grouped key/value heads
        (k, v with H_kv heads dividing H) and, forward and backward, a causal
        sliding window (window=w: key j visible to query i iff i - w < j <= i)
    fa_bwd_workspace_bytes(B, H, N, d), fa_decode_workspace_bytes(B, H, d, S)
    fa_status_string(code), fa_version()
Convenience wrappers allocate outputs and workspaces with torch:
    attention_fwd, attention_bwd, attention_decode
and attention(q, k, v, scale=None, causal=False, window=0) is a differentiable
drop-in for torch's scaled_dot_product_attention on [B, H, N, d] fp16/bf16
device tensors (the PyTorch entry point the pages name: "FlashAttention
ontleed", § "Praktische integratie en hardware-eisen"; "03. FlashAttention",
§ "Intégration en pratique"): its forward saves O and the log-sum-exp and its
backward recomputes P through fa_bwd ("03. FlashAttention", § "Backward pass").
"""
import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libfa.so")

FA_OK = 0
FA_F16, FA_BF16 = 0, 1
FA_MAX_SPLITS = 256
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_DTYPE",
                4: "FA_ERR_ALIGN", 5: "FA_ERR_UNSUPPORTED", 6: "FA_ERR_WORKSPACE",
                7: "FA_ERR_HIP", 8: "FA_ERR_SPLITS", 9: "FA_ERR_SCRATCH"}
FA_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_status_string(code)}")


def load_library(path: str = LIB_PATH):
    """Load libfa.so and declare its C signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m exact_io_aware_31_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, i, vp]
    lib.fa_decode.restype = i
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i,
                              i, vp]
    lib.fa_bwd_ex.restype = i
    lib.fa_decode_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, i, vp]
    lib.fa_decode_ex.restype = i
    lib.fa_decode_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, i, vp]
    lib.fa_decode_varlen.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def fa_version() -> str:
    return load_library().fa_version().decode()


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d))


def fa_decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, H, d, num_splits))


# ------------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _dt_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; use float16 or bfloat16")


def _dev(t, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(code: int, where: str):
    if code != FA_OK:
        raise FAError(code, where)


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    """Enqueue the fused forward: o, lse <- attention(q, k, v)."""
    torch = _torch()
    B, H, N, d = q.shape
    args = [_dev(q, "q"), _dev(k, "k", q.dtype, q.shape), _dev(v, "v", q.dtype, q.shape),
            _dev(o, "o", q.dtype, q.shape), _dev(lse, "lse", torch.float32, (B, H, N))]
    _check(load_library().fa_fwd(*args, B, H, N, d, float(scale), int(bool(causal)),
                                 _dt_code(q), _stream(q, stream)), "fa_fwd")


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale: float, causal: bool,
           stream=None):
    """Enqueue the backward: dq, dk, dv <- gradients for upstream gradient dout."""
    torch = _torch()
    B, H, N, d = q.shape
    sh = q.shape
    args = [_dev(q, "q"), _dev(k, "k", q.dtype, sh), _dev(v, "v", q.dtype, sh),
            _dev(o, "o", q.dtype, sh), _dev(lse, "lse", torch.float32, (B, H, N)),
            _dev(dout, "dout", q.dtype, sh), _dev(dq, "dq", q.dtype, sh),
            _dev(dk, "dk", q.dtype, sh), _dev(dv, "dv", q.dtype, sh), _dev(workspace, "workspace")]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd(*args, nbytes, B, H, N, d, float(scale), int(bool(causal)),
                                 _dt_code(q), _stream(q, stream)), "fa_bwd")


def fa_decode(q, k, v, o, lse, scale: float, num_splits: int, workspace, stream=None):
    """Enqueue split-history decode: q [B,H,1,d], k/v [B,H,Nkv,d] -> o [B,H,1,d], lse [B,H]."""
    torch = _torch()
    B, H, Nkv, d = k.shape
    args = [_dev(q, "q", k.dtype, (B, H, 1, d)), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
            _dev(o, "o", k.dtype, (B, H, 1, d)),
            _dev(lse, "lse", torch.float32, (B, H)) if lse is not None else ctypes.c_void_p(0)]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_decode(*args, B, H, Nkv, d, float(scale), int(num_splits),
                                    _dev(workspace, "workspace"), nbytes, _dt_code(k),
                                    _stream(k, stream)), "fa_decode")


def _kv_heads(q, k) -> int:
    B, H = q.shape[0], q.shape[1]
    if k.dim() != 4 or k.shape[0] != B or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"k has shape {tuple(k.shape)}; expected [B, H_kv, N, d] for q "
                         f"{tuple(q.shape)}")
    hkv = k.shape[1]
    if hkv < 1 or H % hkv != 0:
        raise ValueError(f"query heads {H} are not a multiple of key/value heads {hkv}")
    return hkv


def fa_fwd_ex(q, k, v, o, lse, scale: float, causal: bool, window: int = 0, stream=None):
    """fa_fwd with k, v of H_kv heads ([B, H_kv, N, d]) and an optional causal window."""
    torch = _torch()
    B, H, N, d = q.shape
    hkv = _kv_heads(q, k)
    kv = (B, hkv, N, d)
    args = [_dev(q, "q"), _dev(k, "k", q.dtype, kv), _dev(v, "v", q.dtype, kv),
            _dev(o, "o", q.dtype, q.shape), _dev(lse, "lse", torch.float32, (B, H, N))]
    _check(load_library().fa_fwd_ex(*args, B, H, hkv, N, d, float(scale), int(bool(causal)),
                                    int(window), _dt_code(q), _stream(q, stream)), "fa_fwd_ex")


def fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale: float, causal: bool,
              window: int = 0, stream=None):
    """fa_bwd with k, v, dk, dv of H_kv heads and an optional causal window."""
    torch = _torch()
    B, H, N, d = q.shape
    hkv = _kv_heads(q, k)
    sh, kv = q.shape, (B, hkv, N, d)
    args = [_dev(q, "q"), _dev(k, "k", q.dtype, kv), _dev(v, "v", q.dtype, kv),
            _dev(o, "o", q.dtype, sh), _dev(lse, "lse", torch.float32, (B, H, N)),
            _dev(dout, "dout", q.dtype, sh), _dev(dq, "dq", q.dtype, sh),
            _dev(dk, "dk", q.dtype, kv), _dev(dv, "dv", q.dtype, kv), _dev(workspace, "workspace")]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_ex(*args, nbytes, B, H, hkv, N, d, float(scale),
                                    int(bool(causal)), int(window), _dt_code(q),
                                    _stream(q, stream)), "fa_bwd_ex")


def fa_decode_ex(q, k, v, o, lse, scale: float, num_splits: int, workspace, stream=None):
    """fa_decode with k, v of H_kv heads: q [B,H,1,d], k/v [B,H_kv,Nkv,d]."""
    torch = _torch()
    B, H, _, d = q.shape
    hkv = _kv_heads(q, k)
    Nkv = k.shape[2]
    args = [_dev(q, "q", k.dtype, (B, H, 1, d)), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
            _dev(o, "o", k.dtype, (B, H, 1, d)),
            _dev(lse, "lse", torch.float32, (B, H)) if lse is not None else ctypes.c_void_p(0)]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_decode_ex(*args, B, H, hkv, Nkv, d, float(scale), int(num_splits),
                                       _dev(workspace, "workspace"), nbytes, _dt_code(k),
                                       _stream(k, stream)), "fa_decode_ex")


def fa_decode_varlen(q, k, v, kv_lens, o, lse, scale: float, num_splits: int, workspace,
                     stream=None):
    """fa_decode_ex over a padded cache of ragged histories: sequence b attends to its first
    kv_lens[b] keys (kv_lens: device int32 [B])."""
    torch = _torch()
    B, H, _, d = q.shape
    hkv = _kv_heads(q, k)
    Nkv = k.shape[2]
    args = [_dev(q, "q", k.dtype, (B, H, 1, d)), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
            _dev(kv_lens, "kv_lens", torch.int32, (B,)), _dev(o, "o", k.dtype, (B, H, 1, d)),
            _dev(lse, "lse", torch.float32, (B, H)) if lse is not None else ctypes.c_void_p(0)]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_decode_varlen(*args, B, H, hkv, Nkv, d, float(scale),
                                           int(num_splits), _dev(workspace, "workspace"), nbytes,
                                           _dt_code(k), _stream(k, stream)), "fa_decode_varlen")


def fa_decode_noalloc(q, k, v, o, lse, scale: float, num_splits: int, stream=None):
    """fa_decode_ex with the per-chunk partials in the library's static device scratch
    (FA_NOALLOC_SCRATCH_BYTES) instead of a caller workspace: q [B,H,1,d], k/v
    [B,H_kv,Nkv,d].  Calls that may run at the same time on one device race."""
    torch = _torch()
    B, H, _, d = q.shape
    hkv = _kv_heads(q, k)
    Nkv = k.shape[2]
    args = [_dev(q, "q", k.dtype, (B, H, 1, d)), _dev(k, "k"), _dev(v, "v", k.dtype, k.shape),
            _dev(o, "o", k.dtype, (B, H, 1, d)),
            _dev(lse, "lse", torch.float32, (B, H)) if lse is not None else ctypes.c_void_p(0)]
    _check(load_library().fa_decode_noalloc(*args, B, H, hkv, Nkv, d, float(scale),
                                            int(num_splits), _dt_code(k), _stream(k, stream)),
           "fa_decode_noalloc")


# ------------------------------------------------------------------ convenience
def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def attention_fwd(q, k, v, scale=None, causal=False, stream=None, window=0):
    """Allocate o and lse and run fa_fwd (fa_fwd_ex when k, v have fewer heads than q or a
    window is given).  Returns (o, lse)."""
    torch = _torch()
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if k.shape[1] != H or window:
        fa_fwd_ex(q, k, v, o, lse, _default_scale(d, scale), causal, window, stream)
    else:
        fa_fwd(q, k, v, o, lse, _default_scale(d, scale), causal, stream)
    return o, lse


def bwd_workspace(q):
    torch = _torch()
    B, H, N, d = q.shape
    return torch.empty(fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)


def decode_workspace(k, num_splits: int, heads=None):
    """Workspace for fa_decode(_ex); heads = query heads (default: k's heads)."""
    torch = _torch()
    B, H, _, d = k.shape
    H = H if heads is None else int(heads)
    return torch.empty(fa_decode_workspace_bytes(B, H, d, num_splits), dtype=torch.uint8,
                       device=k.device)


def attention_bwd(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None,
                  window=0):
    """Allocate gradients (and workspace if not given) and run fa_bwd (fa_bwd_ex for grouped
    heads or a window).  Returns (dq, dk, dv)."""
    torch = _torch()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = bwd_workspace(q) if workspace is None else workspace
    sc = _default_scale(q.shape[-1], scale)
    if k.shape[1] != q.shape[1] or window:
        fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, ws, sc, causal, window, stream)
    else:
        fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, sc, causal, stream)
    return dq, dk, dv


def attention_decode(q, k, v, scale=None, num_splits=16, workspace=None, stream=None,
                     kv_lens=None):
    """Allocate o, lse (and workspace if not given) and run fa_decode (fa_decode_ex when k, v
    have fewer heads than q; fa_decode_varlen when kv_lens, a device int32 [B] of history
    lengths, is given).  Returns (o, lse)."""
    torch = _torch()
    B, H, _, d = q.shape
    o = torch.empty((B, H, 1, d), dtype=k.dtype, device=k.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=k.device)
    ws = decode_workspace(k, num_splits, heads=H) if workspace is None else workspace
    if kv_lens is not None:
        fa_decode_varlen(q, k, v, kv_lens, o, lse, _default_scale(d, scale), num_splits, ws,
                         stream)
    elif k.shape[1] != H:
        fa_decode_ex(q, k, v, o, lse, _default_scale(d, scale), num_splits, ws, stream)
    else:
        fa_decode(q, k, v, o, lse, _default_scale(d, scale), num_splits, ws, stream)
    return o, lse


# ------------------------------------------------------------------ autograd
_Function = None


def _function():
    """The autograd.Function, built on first use (torch is imported lazily)."""
    global _Function
    if _Function is not None:
        return _Function
    torch = _torch()

    class FlashAttentionFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, scale, causal, window):
            o, lse = attention_fwd(q, k, v, scale, causal, window=window)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.scale, ctx.causal, ctx.window = scale, causal, window
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = attention_bwd(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal,
                                       window=ctx.window)
            return dq, dk, dv, None, None, None

    _Function = FlashAttentionFunction
    return _Function


def attention(q, k, v, scale=None, causal=False, window=0):
    """Differentiable exact attention: softmax(scale q k^T [causal, window]) v.

    q [B, H, N, d], k and v [B, H_kv, N, d] (H_kv dividing H), fp16 or bf16,
    contiguous device tensors; scale defaults to 1/sqrt(d).  The same result
    as torch.nn.functional.scaled_dot_product_attention(q, k, v,
    is_causal=causal, scale=scale, enable_gqa=True) up to rounding, computed
    by libfa's kernels in both directions."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    return _function().apply(q.contiguous(), k.contiguous(), v.contiguous(),
                             _default_scale(q.shape[-1], scale), bool(causal), int(window))
