"""The largest sizes the C ABI accepts, on the GPU against the float64 oracle.

* Forward and backward on tensors of more than 2^31 elements (B2 H4224 N2048 d128 bf16,
  4.4 GB each): the (batch, head) base offsets no longer fit 32 bits.  Every output element
  must be written (outputs start as NaN), and whole heads are checked against the oracle on
  both sides of the 2^31-element boundary and at the far end.
* Decode over a history of 2^24 - 1 keys at d = 128: N_kv d = 2^31 - 128, the largest
  per-head extent the ABI accepts (one more key is refused).  The reference is the oracle's
  decode on consecutive slices of the history, merged with the oracle's log-sum-exp merge
  (pinned against the unsplit decode on the CPU), so the host never holds the whole history
  in float64.
Inputs are drawn on the GPU from a seeded generator; the oracle receives the exact bits.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import (announce, check_max_abs, check_rel_norm, check_rel_norm_blocks,
                               host64, nan_like)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_fwd_bwd_beyond_2_31_elements():
    B, H, N, d, dtype = 2, 4224, 2048, 128, torch.bfloat16
    seed = 9400
    assert B * H * N * d > 2 ** 31
    announce(f"large fwd+bwd B{B} H{H} N{N} d{d} causal ({B * H * N * d} elements) seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, DEV, with_dout=True)
    scale = d ** -0.5
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, scale, True)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, fa.bwd_workspace(q), scale, True)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name}: unwritten or non-finite elements"
    # heads (b, h): the first, both sides of the 2^31-element boundary, and the last
    edge = 2 ** 31 // (N * d)
    heads = {(0, 0), divmod(edge - 1, H), divmod(edge, H), (B - 1, H - 1)}
    for b, h in sorted(heads):
        qh, kh, vh, doh = (t[b, h].cpu() for t in (q, k, v, do))
        o_ref, lse_ref = oracle.attn_fwd(qh, kh, vh, scale, True)
        check_max_abs(host64(o[b, h]), o_ref, dtype, f"O head ({b},{h})")
        check_max_abs(host64(lse[b, h]), lse_ref, dtype, f"lse head ({b},{h})")
        ref = oracle.attn_bwd(qh, kh, vh, doh, scale, True)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_rel_norm(host64(g[b, h]), r, dtype, f"{name} head ({b},{h})")
            check_rel_norm_blocks(host64(g[b, h]), r, dtype, f"{name} head ({b},{h})")


def test_decode_longest_history_the_abi_accepts():
    B, H, Hkv, d, dtype, splits = 1, 4, 1, 128, torch.bfloat16, 256
    Nkv = 2 ** 31 // d - 1
    seed = 9401
    announce(f"decode B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, DEV, Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    o = nan_like(q)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    ws = fa.decode_workspace(k, splits, heads=H)
    fa.fa_decode_ex(q, k, v, o, lse, scale, splits, ws)
    torch.cuda.synchronize()
    # one key more is refused
    k1 = torch.empty((1, 1, Nkv + 1, d), dtype=dtype, device=DEV)
    with pytest.raises(fa.FAError) as err:
        fa.fa_decode_ex(q, k1, k1, o.clone(), lse.clone(), scale, splits, ws)
    assert fa.STATUS_NAMES[err.value.code] == "FA_ERR_SHAPE"
    del k1
    # reference: the oracle on 16 consecutive slices of the history, merged per head
    qh = q.cpu()
    parts_o, parts_lse = [], []
    bounds = np.linspace(0, Nkv, 17).astype(np.int64)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o_c, lse_c = oracle.attn_decode(qh, k[:, :, lo:hi].cpu(), v[:, :, lo:hi].cpu(), scale)
        parts_o.append(o_c.reshape(H, d))
        parts_lse.append(lse_c.reshape(H))
    o_h, lse_h = host64(o).reshape(H, d), host64(lse).reshape(H)
    for h in range(H):
        o_ref, lse_ref = oracle.lse_merge(np.stack([p[h] for p in parts_o]),
                                          np.array([p[h] for p in parts_lse]))
        check_max_abs(o_h[h], o_ref, dtype, f"O head {h}")
        check_max_abs(lse_h[h:h + 1], np.array([lse_ref]), dtype, f"lse head {h}")
