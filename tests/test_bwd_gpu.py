"""GPU parity of fa_bwd against the float64 oracle (called through the C ABI).

The GPU backward consumes the O and lse written by the GPU forward (as a
training step would); the oracle recomputes everything in float64 from Q, K,
V and dO.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import BWD_4K, attention_inputs
from tests.parity_util import announce, check_rel_norm, check_rel_norm_blocks, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_fwd_bwd(q, k, v, do, scale, causal):
    o, lse = fa.attention_fwd(q, k, v, scale, causal)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    ws = fa.bwd_workspace(q)
    ws.fill_(0xFF)  # garbage in: the workspace contents on entry must not matter
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1, 17, 64, 130, 257])
def test_bwd_sweep(N, causal, d, dtype):
    B, H = 1, 2
    seed = 8000 + N + 13 * d + (1 if causal else 0)
    announce(f"bwd sweep B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True)
    scale = d ** -0.5
    got = run_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)), scale, causal)
    ref = oracle.attn_bwd(q, k, v, do, scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        check_rel_norm(host64(g), r, dtype, name)


def test_bwd_full_size_workload():
    w = BWD_4K
    announce(f"bwd {w.name} seed={w.seed} (inputs drawn on the host)")
    q, k, v, do = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, "cpu", with_dout=True)
    dq, dk, dv = run_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)), w.scale, w.causal)
    # properties of every head: rows of dS sum to 0, rows of P sum to 1
    dk32, dv32, do32 = dk.float(), dv.float(), do.to(DEV).float()
    colsum_dk = dk32.sum(dim=2)
    assert float(colsum_dk.abs().max()) <= 5e-2 * float(dk32.abs().sum(dim=2).max())
    diff_dv = (dv32.sum(dim=2) - do32.sum(dim=2)).abs().max()
    assert float(diff_dv) <= 5e-2 * float(do32.abs().sum(dim=2).max())
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        ref = oracle.attn_bwd(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_rel_norm(host64(g[b, h]), r, w.dtype, f"{name} head ({b},{h})")
            check_rel_norm_blocks(host64(g[b, h]), r, w.dtype, f"{name} head ({b},{h})")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_many_heads(causal, d, dtype):
    """A grid of several workgroups per CU in both passes (512 heads); N = 500 leaves a ragged
    last key block (dK/dV pass) and a ragged last query block (dQ pass)."""
    B, H, N = 2, 256, 500
    seed = 8500 + d + (1 if causal else 0)
    announce(f"bwd wide blocks B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True)
    scale = d ** -0.5
    dq, dk, dv = run_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)), scale, causal)
    for b, h in [(0, 0), (0, 131), (1, 255)]:
        ref = oracle.attn_bwd(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_rel_norm(host64(g[b, h]), r, dtype, f"{name} head ({b},{h})")
            check_rel_norm_blocks(host64(g[b, h]), r, dtype, f"{name} head ({b},{h})")


def test_bwd_at_bench_shape():
    """The backward launch the benchmark times: B1 H32 N8192 d128 bf16 causal, Q x2."""
    from synth_inputs import FWD_8K as w
    announce(f"bwd at the benchmark shape {w.name} seed={w.seed}")
    q, k, v, do = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, "cpu", q_mult=w.q_mult,
                                   with_dout=True)
    dq, dk, dv = run_fwd_bwd(*(t.to(DEV) for t in (q, k, v, do)), w.scale, w.causal)
    for b, h in [(0, 0), (0, w.H - 1)]:
        ref = oracle.attn_bwd(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_rel_norm(host64(g[b, h]), r, w.dtype, f"{name} head ({b},{h})")
            check_rel_norm_blocks(host64(g[b, h]), r, w.dtype, f"{name} head ({b},{h})")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_deterministic(causal):
    """Every gradient element is written once by one lane (no atomics): repeated calls on the
    same inputs give bitwise-equal dQ, dK and dV."""
    B, H, N, d, dtype = 2, 8, 1000, 128, torch.bfloat16
    seed = 8700 + (1 if causal else 0)
    announce(f"bwd determinism B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, DEV, with_dout=True)
    scale = d ** -0.5
    first = run_fwd_bwd(q, k, v, do, scale, causal)
    for _ in range(2):
        again = run_fwd_bwd(q, k, v, do, scale, causal)
        for name, a, b in zip(("dQ", "dK", "dV"), first, again):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs between runs"


@pytest.mark.parametrize("B,H,Hkv,N,causal,d,dtype", [
    (1, 2, 2, 4096, True, 128, torch.bfloat16),    # 128 blocks of 64 keys: steps split in 2
    (1, 2, 2, 4160, False, 128, torch.bfloat16),   # 130 blocks of 64 keys: not split
    (1, 4, 4, 2048, True, 128, torch.bfloat16),    # 128 blocks of 64, 256 of 32: split in 2
    (1, 8, 4, 2048, False, 64, torch.float16),     # grouped heads, split in 2
    (1, 8, 2, 2048, True, 128, torch.bfloat16),    # 128 blocks of 32 keys: split in 4
    (1, 3, 3, 1111, False, 64, torch.float16),     # ragged end, odd step counts, split in 4
    (2, 16, 4, 2048, True, 128, torch.bfloat16),   # grouped, 256 blocks of 64 keys: split in 2
    (1, 16, 4, 2048, True, 128, torch.bfloat16),   # grouped, 256 blocks of 32 keys: split in 4
    (1, 4, 4, 4096, True, 64, torch.bfloat16),     # d = 64, 256 blocks of 64 keys: split in 2
], ids=["split2-128", "nosplit-130", "split2-small", "split2-grouped", "split4-grouped",
        "split4-f16-d64-ragged", "split2-grouped-256", "split4-grouped-256", "split2-d64-256"])
def test_bwd_query_split_boundary(B, H, Hkv, N, causal, d, dtype):
    """Grids of at most 128 blocks of 32 keys (256 with grouped heads) run the dK/dV pass with
    four waves per block of 32 keys, each taking every fourth query step; else, grids of at
    most 128 blocks of 64 keys (256 with grouped heads or d = 64) with two pairs of waves per
    block taking the even and the odd steps.  The waves merge dK and dV at the end.  Key/value
    groups against the oracle (at most three per case), whole tensor and every 32-row block."""
    seed = 8600 + N + H + Hkv + d + (1 if causal else 0)
    announce(f"bwd query split B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True, Hkv=Hkv)
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.attention_fwd(qd, kd, vd, scale, causal)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale, causal)
    torch.cuda.synchronize()
    dq_h, dk_h, dv_h = host64(dq), host64(dk), host64(dv)
    g = H // Hkv
    groups = sorted({(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)})
    for b, hk in groups:
        hs = slice(g * hk, g * hk + g)
        ref = oracle.attn_bwd(q[b, hs], k[b, hk:hk + 1], v[b, hk:hk + 1], do[b, hs], scale, causal)
        for name, gt, r in (("dQ", dq_h[b, hs], ref[0]), ("dK", dk_h[b, hk:hk + 1], ref[1]),
                            ("dV", dv_h[b, hk:hk + 1], ref[2])):
            check_rel_norm(gt, r, dtype, f"{name} group ({b},{hk})")
            check_rel_norm_blocks(gt, r, dtype, f"{name} group ({b},{hk})")
