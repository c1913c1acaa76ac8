"""Float64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The HIP library never imports,
links or calls it, and it imports nothing from the HIP package.

Thin ctypes wrapper over ``oracle.c`` (plain C, float64, OpenMP): every
function here only marshals arrays; the arithmetic is in the C file, where
each function cites the passage of the pages it follows.  Inputs may be
numpy arrays or torch tensors of any float dtype; they are widened exactly
to float64 (fp16 and bf16 values are exactly representable in float64).

Shapes follow the attention problem statement: q, k, v are [..., N, d]
(leading dims are flattened into independent heads).  Grouped key/value
heads: q [..., H, N, d] with k, v [..., H_kv, N, d], H a multiple of H_kv;
query head h reads key/value head h // (H / H_kv).

Parity status: every function is pinned by tests/test_oracle.py against
values printed on the pages, closed forms, invariants, finite differences
and an independent library routine; none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # A mutation test may point the wrapper at a deliberately broken copy.
    path = os.environ.get("ORACLE_LIB_OVERRIDE") or _build.LIB
    if path == _build.LIB and ((not os.path.exists(path)) or
                               os.path.getmtime(_build.SRC) > os.path.getmtime(path)):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_softmax.argtypes = [_dp, ctypes.c_long, _dp]
    lib.oracle_softmax.restype = None
    lib.oracle_softmax_online.argtypes = [_dp, ctypes.c_long, ctypes.c_long, _dp, _dp, _dp]
    lib.oracle_softmax_online.restype = ctypes.c_long
    lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_long,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                    ctypes.c_int, _lp, ctypes.c_int]
    lib.oracle_attn_fwd.restype = ctypes.c_int
    lib.oracle_attn_decode.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_long,
                                       ctypes.c_long, ctypes.c_double, ctypes.c_int]
    lib.oracle_attn_decode.restype = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_attn_fwd_w.argtypes = [_dp, _dp, _dp, _dp, _dp, L, L, L, L, L, L, ctypes.c_double,
                                      ctypes.c_int, L, _lp, ctypes.c_int]
    lib.oracle_attn_fwd_w.restype = ctypes.c_int
    lib.oracle_attn_decode_w.argtypes = [_dp, _dp, _dp, _dp, _dp, L, L, L, L, L, ctypes.c_double,
                                         ctypes.c_int]
    lib.oracle_attn_decode_w.restype = ctypes.c_int
    lib.oracle_attn_bwd_w.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, L, L, L, L, L,
                                      ctypes.c_double, ctypes.c_int, L, ctypes.c_int]
    lib.oracle_attn_bwd_w.restype = ctypes.c_int
    lib.oracle_attn_fwd_tiled.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_long,
                                          ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                          ctypes.c_int, ctypes.c_long, ctypes.c_long]
    lib.oracle_attn_fwd_tiled.restype = ctypes.c_int
    lib.oracle_lse_merge.argtypes = [_dp, _dp, ctypes.c_long, ctypes.c_long, _dp, _dp]
    lib.oracle_lse_merge.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_long,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                    ctypes.c_int, ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Exact widening to a C-contiguous float64 numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def max_threads() -> int:
    """OpenMP threads the oracle's parallel regions use."""
    return int(_load().oracle_max_threads())


def softmax(x):
    """Softmax of a 1-D row by definition (max subtracted first)."""
    x = _f64(x).reshape(-1)
    p = np.empty_like(x)
    _load().oracle_softmax(_ptr(x), x.size, _ptr(p))
    return p


def softmax_online(x, chunk: int):
    """Chunked one-pass softmax; returns (p, m_trace, l_trace) per chunk."""
    x = _f64(x).reshape(-1)
    n = x.size
    nch = max(1, -(-n // int(chunk)))
    p = np.empty_like(x)
    mt = np.empty(nch)
    lt = np.empty(nch)
    got = _load().oracle_softmax_online(_ptr(x), n, int(chunk), _ptr(p), _ptr(mt), _ptr(lt))
    return p, mt[:got], lt[:got]


def _heads(qlead, klead):
    """(B, H, H_kv) for leading dims of q [..., H, ., d] and k [..., H_kv, ., d]."""
    if tuple(qlead) == tuple(klead):
        bh = int(np.prod(qlead)) if qlead else 1
        return 1, bh, bh
    assert len(qlead) >= 1 and tuple(qlead[:-1]) == tuple(klead[:-1]), "batch dims differ"
    assert qlead[-1] % klead[-1] == 0, "query heads must be a multiple of key/value heads"
    return int(np.prod(qlead[:-1])) if len(qlead) > 1 else 1, int(qlead[-1]), int(klead[-1])


def attn_fwd(q, k, v, scale: float, causal: bool, qpos=None, nthreads: int = 0,
             window: int = 0):
    """Three-step attention.  q [..., nq, d], k/v [..., nk, d] -> (o, lse).

    window > 0 (with causal): key j visible to query i iff i - window < j <= i.
    k and v may have fewer heads than q (grouped-query attention)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    nq, d = q.shape[-2:]
    nk = k.shape[-2]
    assert v.shape == k.shape and k.shape[-1] == d
    b, h, hkv = _heads(lead, k.shape[:-2])
    o = np.empty(q.shape)
    lse = np.empty(lead + (nq,))
    qp = None
    if qpos is not None:
        qp_arr = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64))
        assert qp_arr.shape == (nq,)
        qp = qp_arr.ctypes.data_as(_lp)
    rc = _load().oracle_attn_fwd_w(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, h, hkv, nq,
                                   nk, d, float(scale), int(bool(causal)), int(window), qp,
                                   int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd_w failed ({rc})")
    return o, lse


def attn_fwd_tiled(q, k, v, scale: float, causal: bool, br: int, bc: int):
    """Tiled forward with online softmax for one head: q [nq, d], k/v [nk, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    o = np.empty((nq, d))
    lse = np.empty(nq)
    rc = _load().oracle_attn_fwd_tiled(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), nq, nk, d,
                                       float(scale), int(bool(causal)), int(br), int(bc))
    if rc != 0:
        raise RuntimeError("oracle_attn_fwd_tiled failed")
    return o, lse


def attn_decode(q, k, v, scale: float, nthreads: int = 0, kv_lens=None):
    """Single-token decode.  q [..., H, d] (or [..., H, 1, d]), k/v [..., H_kv, nkv, d]
    (H_kv may divide H); returns o [..., H, d] and lse [..., H].

    kv_lens (q, k, v of shape [B, H, 1, d] / [B, H_kv, nkv, d]): sequence b attends
    to its first kv_lens[b] keys only (a padded cache of ragged histories); a
    sequence with no keys gets o = 0, lse = -inf."""
    if kv_lens is not None:
        q, k, v = _f64(q), _f64(k), _f64(v)
        lens = [int(x) for x in np.asarray(kv_lens).reshape(-1)]
        assert k.ndim == 4 and len(lens) == k.shape[0]
        outs = [attn_decode(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], scale,
                            nthreads) for b in range(k.shape[0])]
        return (np.concatenate([o for o, _ in outs]), np.concatenate([l for _, l in outs]))
    q, k, v = _f64(q), _f64(k), _f64(v)
    nkv, d = k.shape[-2:]
    klead = k.shape[:-2]
    if k.ndim >= 3:
        batch, hkv = klead[:-1], int(klead[-1])
    else:
        batch, hkv = (), 1
    b = int(np.prod(batch)) if batch else 1
    h = q.size // d // b
    assert h * b * d == q.size and h % hkv == 0
    q = q.reshape(b * h, d)
    o = np.empty(batch + (h, d)) if k.ndim >= 3 else np.empty((d,))
    lse = np.empty(batch + (h,)) if k.ndim >= 3 else np.empty(())
    rc = _load().oracle_attn_decode_w(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, h, hkv,
                                      nkv, d, float(scale), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_decode_w failed ({rc})")
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge per-chunk (o_c [nparts, d], lse_c [nparts]) of one row."""
    op, lp = _f64(o_parts), _f64(lse_parts).reshape(-1)
    nparts, d = op.shape
    o = np.empty(d)
    lse = np.empty(1)
    rc = _load().oracle_lse_merge(_ptr(op), _ptr(lp), nparts, d, _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_lse_merge failed")
    return o, float(lse[0])


def attn_bwd(q, k, v, dout, scale: float, causal: bool, return_drow: bool = False,
             nthreads: int = 0, window: int = 0):
    """Gradients of the three-step definition.  q, dout [..., n, d]; k, v [..., n, d]
    with possibly fewer heads than q (their gradients sum over each group)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    assert v.shape == k.shape and k.shape[-2:] == (n, d) and do.shape == q.shape
    b, h, hkv = _heads(lead, k.shape[:-2])
    dq, dk, dv = np.empty(q.shape), np.empty(k.shape), np.empty(k.shape)
    drow = np.empty(lead + (n,))
    rc = _load().oracle_attn_bwd_w(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(drow), b, h, hkv, n, d, float(scale),
                                   int(bool(causal)), int(window), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd_w failed ({rc})")
    if return_drow:
        return dq, dk, dv, drow
    return dq, dk, dv
