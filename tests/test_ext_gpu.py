"""GPU parity of fa_fwd_ex / fa_bwd_ex / fa_decode_ex (grouped key/value heads and a
causal sliding window) against the float64 oracle, through the C ABI.

Grouped heads: k and v have H_kv heads, query head h reads head h / (H / H_kv), and
dk, dv sum over each group.  Window w: key j is visible to query i iff i - w < j <= i.
Tolerances are those of the plain entry points (tests/parity_util.py).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_max_abs, check_rel_norm, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_fwd_ex(q, k, v, scale, causal, window):
    B, H, N, d = q.shape
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd_ex(q, k, v, o, lse, scale, causal, window)
    torch.cuda.synchronize()
    return o, lse


def run_bwd_ex(q, k, v, do, scale, causal, window):
    o, lse = run_fwd_ex(q, k, v, scale, causal, window)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    ws = fa.bwd_workspace(q)
    ws.fill_(0xFF)
    fa.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal, window)
    torch.cuda.synchronize()
    return dq, dk, dv


FWD_CASES = [  # (B, H, H_kv, N, window)
    (2, 4, 2, 130, 0), (1, 8, 1, 257, 0), (2, 6, 3, 64, 0),
    (1, 4, 4, 300, 1), (2, 4, 2, 257, 17), (1, 4, 1, 1000, 64), (1, 2, 2, 1000, 100),
    (1, 8, 2, 777, 300), (1, 2, 1, 200, 199),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,N,window", FWD_CASES)
def test_fwd_ex(B, H, Hkv, N, window, d, dtype):
    causal = True if window else (N % 2 == 0)
    seed = 9000 + N + H + 7 * Hkv + window + d
    announce(f"fwd_ex B{B} H{H} Hkv{Hkv} N{N} d{d} window={window} causal={causal} {dtype} "
             f"seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu", Hkv=Hkv)
    scale = d ** -0.5
    o, lse = run_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal, window)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal, window=window)
    check_max_abs(host64(o), o_ref, dtype, "O")
    check_max_abs(host64(lse), lse_ref, dtype, "lse")


BWD_CASES = [  # (B, H, H_kv, N, window)
    (2, 4, 2, 130, 0), (1, 8, 1, 257, 0), (1, 4, 4, 300, 1), (2, 4, 2, 257, 17),
    (1, 4, 1, 700, 64), (1, 6, 3, 500, 200), (1, 2, 2, 260, 259),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,N,window", BWD_CASES)
def test_bwd_ex(B, H, Hkv, N, window, d, dtype):
    causal = True if window else (N % 2 == 1)
    seed = 9500 + N + H + 7 * Hkv + window + d
    announce(f"bwd_ex B{B} H{H} Hkv{Hkv} N{N} d{d} window={window} causal={causal} {dtype} "
             f"seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True, Hkv=Hkv)
    scale = d ** -0.5
    got = run_bwd_ex(*(t.to(DEV) for t in (q, k, v, do)), scale, causal, window)
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window=window)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        check_rel_norm(host64(g), r, dtype, name)


def test_ex_without_groups_or_window_is_the_plain_call():
    """fa_fwd_ex / fa_bwd_ex with H_kv = H and window 0 (or a window covering the sequence)
    run the same kernels as fa_fwd / fa_bwd: bitwise-equal results."""
    B, H, N, d, dtype = 1, 4, 333, 128, torch.bfloat16
    announce(f"ex == plain B{B} H{H} N{N} d{d}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, 9901, DEV, with_dout=True)
    scale = d ** -0.5
    for window in (0, N, N + 50):
        o1, l1 = run_fwd_ex(q, k, v, scale, True, window)
        o2, l2 = fa.attention_fwd(q, k, v, scale, True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        g1 = run_bwd_ex(q, k, v, do, scale, True, window)
        g2 = fa.attention_bwd(q, k, v, o2, l2, do, scale, True)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_bwd_ex_grouped_is_deterministic():
    B, H, Hkv, N, d = 1, 8, 2, 600, 128
    announce(f"bwd_ex determinism B{B} H{H} Hkv{Hkv} N{N}")
    q, k, v, do = attention_inputs(B, H, N, d, torch.bfloat16, 9902, DEV, with_dout=True, Hkv=Hkv)
    first = run_bwd_ex(q, k, v, do, d ** -0.5, True, 77)
    again = run_bwd_ex(q, k, v, do, d ** -0.5, True, 77)
    for a, b in zip(first, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,Nkv,splits", [(2, 8, 2, 1000, 4), (3, 4, 1, 333, 16),
                                                (1, 6, 3, 64, 3), (2, 4, 4, 257, 1)])
def test_decode_ex(B, H, Hkv, Nkv, splits, d, dtype):
    seed = 9700 + Nkv + H + Hkv + d
    announce(f"decode_ex B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = nan_like(qd)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    ws = fa.decode_workspace(kd, splits, heads=H)
    ws.fill_(0xFF)
    fa.fa_decode_ex(qd, kd, vd, o, lse, scale, splits, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(q, k, v, scale)
    check_max_abs(host64(o)[:, :, 0], o_ref, dtype, "O")
    check_max_abs(host64(lse), lse_ref, dtype, "lse")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hkv,splits", [(2, 4), (8, 16), (1, 1)])
def test_decode_varlen(Hkv, splits, d, dtype):
    B, H, Nkv = 6, 8, 700
    lens = [700, 1, 0, 333, 64, 699]
    seed = 9750 + Hkv + splits + d
    announce(f"decode_varlen B{B} H{H} Hkv{Hkv} Nkv{Nkv} lens={lens} d{d} splits={splits} "
             f"{dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = nan_like(qd)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    ws = fa.decode_workspace(kd, splits, heads=H)
    ws.fill_(0xFF)
    fa.fa_decode_varlen(qd, kd, vd, kv_lens, o, lse, scale, splits, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(q, k, v, scale, kv_lens=lens)
    got_o, got_lse = host64(o)[:, :, 0], host64(lse)
    for b, n in enumerate(lens):
        if n == 0:  # no keys: o = 0, lse = -inf
            assert not np.any(got_o[b]) and np.all(got_lse[b] == -np.inf)
            continue
        check_max_abs(got_o[b], o_ref[b], dtype, f"O seq {b} (len {n})")
        check_max_abs(got_lse[b], lse_ref[b], dtype, f"lse seq {b} (len {n})")


@pytest.mark.parametrize("B,H,N,window", [(4, 60, 1024, 300), (2, 64, 2304, 2100)],
                         ids=["4wave", "8wave"])
def test_fwd_ex_both_workgroup_shapes(B, H, N, window):
    """Grouped heads and a window: windows up to 2048 keys run four-wave workgroups; a
    2100-key window over 1152 blocks of 256 rows runs eight-wave ones."""
    d, dtype = 128, torch.bfloat16
    Hkv = H // 4
    seed = 9950 + H
    announce(f"fwd_ex shapes B{B} H{H} Hkv{Hkv} N{N} d{d} window={window} seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu", Hkv=Hkv)
    scale = d ** -0.5
    o, lse = run_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), scale, True, window)
    o_h, lse_h = host64(o), host64(lse)
    for b, h in [(0, 0), (B // 2, H // 2 + 1), (B - 1, H - 1)]:
        hk = h // (H // Hkv)
        o_ref, lse_ref = oracle.attn_fwd(q[b, h], k[b, hk], v[b, hk], scale, True, window=window)
        check_max_abs(o_h[b, h], o_ref, dtype, f"O head ({b},{h})")
        check_max_abs(lse_h[b, h], lse_ref, dtype, f"lse head ({b},{h})")


@pytest.mark.parametrize("B,H,N,window", [(2, 28, 1024, 300), (2, 32, 2304, 2100),
                                          (2, 64, 2304, 2100)],
                         ids=["4wave-dq", "8wave-dq", "4wave-dq-large"])
def test_bwd_ex_both_dq_shapes(B, H, N, window):
    """Grouped heads and a window in the backward at dQ grids of 224 (four-wave workgroups),
    576 (eight-wave) and 1152 (four-wave) blocks of 256 rows: the dQ pass runs four-wave
    workgroups below 256 blocks and from 1024 on.  Whole key/value groups against the oracle."""
    d, dtype = 128, torch.bfloat16
    Hkv = H // 4
    seed = 9960 + H
    announce(f"bwd_ex shapes B{B} H{H} Hkv{Hkv} N{N} d{d} window={window} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True, Hkv=Hkv)
    scale = d ** -0.5
    dq, dk, dv = run_bwd_ex(*(t.to(DEV) for t in (q, k, v, do)), scale, True, window)
    dq_h, dk_h, dv_h = host64(dq), host64(dk), host64(dv)
    for b, hk in [(0, 0), (B - 1, Hkv - 1)]:
        hs = slice(4 * hk, 4 * hk + 4)
        ref = oracle.attn_bwd(q[b, hs], k[b, hk:hk + 1], v[b, hk:hk + 1], do[b, hs], scale, True,
                              window=window)
        check_rel_norm(dq_h[b, hs], ref[0], dtype, f"dQ group ({b},{hk})")
        check_rel_norm(dk_h[b, hk:hk + 1], ref[1], dtype, f"dK head ({b},{hk})")
        check_rel_norm(dv_h[b, hk:hk + 1], ref[2], dtype, f"dV head ({b},{hk})")
