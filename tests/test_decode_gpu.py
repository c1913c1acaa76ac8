"""GPU parity of fa_decode against the float64 oracle (called through the C ABI)."""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import DECODE_16K, attention_inputs
from tests.parity_util import announce, check_max_abs, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_decode(q, k, v, scale, splits):
    B, H, _, d = k.shape
    o = torch.full((B, H, 1, d), float("nan"), dtype=k.dtype, device=k.device)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=k.device)
    ws = fa.decode_workspace(k, splits)
    ws.fill_(0xFF)
    fa.fa_decode(q, k, v, o, lse, scale, splits, ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 3, 16])
@pytest.mark.parametrize("nkv", [1, 5, 100, 1000, 1025, 3000])
def test_decode_sweep(nkv, splits, d, dtype):
    B, H = 2, 3
    seed = 9000 + nkv + 7 * splits + d
    announce(f"decode sweep B{B} H{H} Nkv{nkv} d{d} splits{splits} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=nkv)
    scale = d ** -0.5
    o, lse = run_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, splits)
    o_ref, lse_ref = oracle.attn_decode(q, k, v, scale)
    check_max_abs(host64(o)[:, :, 0], o_ref, dtype, "O")
    check_max_abs(host64(lse), lse_ref, dtype, "lse")


def test_decode_without_lse_output():
    announce("decode with lse=NULL")
    q, k, v = (t.to(DEV) for t in attention_inputs(1, 2, 1, 128, torch.bfloat16, 5, "cpu", Nkv=777))
    o = torch.empty(1, 2, 1, 128, dtype=torch.bfloat16, device=DEV)
    ws = fa.decode_workspace(k, 4)
    fa.fa_decode(q, k, v, o, None, 128 ** -0.5, 4, ws)
    o2, _ = run_decode(q, k, v, 128 ** -0.5, 4)
    assert torch.equal(o, o2)


def test_decode_full_size_workload():
    """Full-size launch (16 GiB of K/V drawn on the GPU); the oracle checks sampled heads."""
    w = DECODE_16K
    announce(f"decode {w.name} seed={w.seed} (inputs drawn on the GPU)")
    q, k, v = attention_inputs(w.B, w.H, 1, w.d, w.dtype, w.seed, DEV, Nkv=w.Nkv)
    o, lse = run_decode(q, k, v, w.scale, w.splits)
    o_h, lse_h = host64(o)[:, :, 0], host64(lse)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h)), "unwritten outputs"
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(b), int(rng.integers(w.H))) for b in
                                            rng.choice(w.B, size=30, replace=False)]
    for b, h in heads:
        o_ref, lse_ref = oracle.attn_decode(q[b, h].cpu(), k[b, h].cpu(), v[b, h].cpu(), w.scale)
        check_max_abs(o_h[b, h], o_ref, w.dtype, f"O head ({b},{h})")
        check_max_abs(np.array(lse_h[b, h]), np.array(lse_ref), w.dtype, f"lse head ({b},{h})")
    del k, v
    torch.cuda.empty_cache()
