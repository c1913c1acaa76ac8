"""The differentiable wrapper exact_io_aware_31_amd.attention (a torch.autograd.Function over
fa_fwd(_ex) / fa_bwd(_ex)) against the float64 oracle."""
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_max_abs, check_rel_norm, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("H,Hkv,causal,window", [(4, 4, False, 0), (4, 4, True, 0), (8, 2, True, 0),
                                                 (4, 1, True, 50), (6, 3, True, 1)])
def test_autograd_matches_oracle(H, Hkv, causal, window):
    B, N, d, dtype = 2, 200, 64, torch.bfloat16
    seed = 9800 + H + Hkv + window
    announce(f"autograd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} window={window} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True, Hkv=Hkv)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = fa.attention(qd, kd, vd, causal=causal, window=window)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    o_ref, _ = oracle.attn_fwd(q, k, v, d ** -0.5, causal, window=window)
    check_max_abs(host64(o), o_ref, dtype, "O")
    ref = oracle.attn_bwd(q, k, v, do, d ** -0.5, causal, window=window)
    for name, t, r in zip(("dQ", "dK", "dV"), (qd, kd, vd), ref):
        assert t.grad.shape == t.shape
        check_rel_norm(host64(t.grad), r, dtype, name)


def test_autograd_in_a_composed_loss():
    """Gradients flow through surrounding torch ops: loss = sum(w * attention(x Wq, x Wk, x Wv))."""
    B, H, N, d = 1, 2, 128, 64
    announce("autograd composed loss")
    g = torch.Generator(device="cpu").manual_seed(9899)
    x = torch.randn(B, H, N, d, generator=g)
    w = torch.randn(B, H, N, d, generator=g)
    wq = (torch.randn(d, d, generator=g) / 8).to(torch.bfloat16)
    xb = x.to(torch.bfloat16)
    q, k, v = (xb @ wq).contiguous(), xb.contiguous(), (xb * 0.5).contiguous()
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    loss = (fa.attention(qd, kd, vd, causal=True).float() * w.to(DEV)).sum()
    loss.backward()
    torch.cuda.synchronize()
    do = w.to(torch.bfloat16).to(torch.float64)  # d loss / d O, as cast back to O's dtype
    ref = oracle.attn_bwd(q, k, v, do, d ** -0.5, True)
    for name, t, r in zip(("dQ", "dK", "dV"), (qd, kd, vd), ref):
        check_rel_norm(host64(t.grad), r, torch.bfloat16, name)
