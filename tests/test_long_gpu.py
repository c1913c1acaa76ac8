"""Long sequences on the GPU against the float64 oracle: a 65 536-token forward (every
K/V tile ring slot reused ~340 times) and a 262 144-key decode history (many sub-chunks of
scores per workgroup), checked on sampled rows / whole heads.  Through the C ABI."""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_max_abs, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("H,causal", [(4, True), (1, False)], ids=["8wave-causal", "4wave-full"])
def test_fwd_long_sequence(H, causal):
    """B1 N65536 d128 bf16: 4 causal heads fill 1024 blocks of 256 rows (eight-wave
    workgroups), 1 non-causal head 256 (four-wave workgroups, two per CU)."""
    B, N, d, dtype = 1, 65536, 128, torch.bfloat16
    seed = 9200 + H
    announce(f"fwd long B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu")
    scale = d ** -0.5
    o = nan_like(q.to(DEV))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, lse, scale, causal)
    torch.cuda.synchronize()
    o_h, lse_h = host64(o), host64(lse)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h)), "unwritten outputs"
    rng = np.random.default_rng(seed)
    for h in range(H):
        rows = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                         rng.choice(N, size=48, replace=False)]))
        o_ref, lse_ref = oracle.attn_fwd(q[0, h, rows], k[0, h], v[0, h], scale, causal,
                                         qpos=rows)
        check_max_abs(o_h[0, h, rows], o_ref, dtype, f"O head {h} rows")
        check_max_abs(lse_h[0, h, rows], lse_ref, dtype, f"lse head {h} rows")


@pytest.mark.parametrize("splits", [16, 256], ids=["16x16384", "256x1024"])
def test_decode_long_history(splits):
    """B1 H8 H_kv2 Nkv262144 d128 bf16: a 16-way split gives 16 384-key chunks (16 score
    sub-chunks per workgroup); 256 chunks is the largest split count."""
    B, H, Hkv, Nkv, d, dtype = 1, 8, 2, 262144, 128, torch.bfloat16
    seed = 9300 + splits
    announce(f"decode long B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} seed={seed}")
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
