"""GPU parity of the forward's rescaling of the partial output when a row's running maximum
grows (Lensa ML explainer, Step 4, online softmax: when a later chunk holds a larger score, the
running sum and the partial output computed so far are scaled down by e^(m_old - m_new)).

The kernel rescales lazily: only when a tile raises a row's maximum by more than 2^8 (in exp2
units) over the reference its probabilities use.  i.i.d. N(0,1) inputs almost never do that
after the first tile, so these inputs add a ramp to the scores: column 0 of Q is a constant a
and column 0 of K rises linearly with the key index, so every row's scores grow steadily along
its visible keys and its maximum passes the slack again and again.  The host first checks that
premise on the exact inputs (in float64, tile by tile as the kernel walks them), then the
kernel's outputs are compared element-wise with the float64 oracle -- for every instantiation
of the forward: bf16 and fp16, d 64 and 128, four- and eight-wave workgroups, non-causal,
causal and a causal window.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_max_abs, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"
SLACK_LOG2 = 8.0   # the kernel's rescale slack, in log2 units
TILE = 64          # keys per tile


def ramp_inputs(B, H, N, d, dtype, seed, a=8.0, top=64.0):
    """N(0,1) inputs with q[..., 0] = a and k[..., j, 0] = top * j / N (rounded to dtype), and V
    halved.  The softmax these scores give is sharp, so an output row is close to a mix of a few
    value rows; halving V keeps |O| below 2, where a bf16 output's own rounding (half an ulp,
    at most 0.0039 there) leaves room for the kernel's rounding of P under the 1e-2 bound (a
    host emulation of both roundings on these inputs gives at most 0.0038, against 0.0076 with
    V unscaled)."""
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu")
    q[..., 0] = a
    k[..., 0] = (torch.arange(N, dtype=torch.float32) * (top / N)).to(dtype)
    v = (v.float() * 0.5).to(dtype)
    return q, k, v


def count_rescales(q, k, scale, causal, window, kbase_of_row):
    """How many times, after the first tile a row sees, a tile raises the row's running maximum
    by more than the slack over the reference kept since the last rescale (float64, log2
    units, tiles of 64 keys from the row's first loaded tile)."""
    q64, k64 = q.double().numpy(), k.double().numpy()
    s = (q64 @ k64.T) * scale * np.log2(np.e)
    n = s.shape[0]
    events = 0
    for i in range(n):
        hi = i + 1 if causal else n
        lo = max(0, i - window + 1) if window else 0
        ref = -np.inf
        first = True
        for t0 in range(kbase_of_row(i), hi, TILE):
            a, b = max(t0, lo), min(t0 + TILE, hi)
            if a >= b:
                continue
            m = s[i, a:b].max()
            if m > ref + SLACK_LOG2:
                events += 0 if first else 1
                ref = m
            first = False
    return events


def run_fwd(q, k, v, scale, causal, window):
    B, H, N, d = q.shape
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    if window:
        fa.fa_fwd_ex(q, k, v, o, lse, scale, causal, window)
    else:
        fa.fa_fwd(q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o, lse


# (mask, workgroup shape) -> (B, H, N, window): without a window, the launcher takes four-wave
# workgroups of 64 rows that split each step's keys between two pairs of waves for at most 256
# blocks of 64 rows (512 at d = 64); four-wave workgroups of 128 rows for at most 256 blocks of 256 query rows,
# for N <= 2048 up to 1024 blocks, and for any window of up to 2048 keys; eight-wave ones
# otherwise.
SHAPES = {("full", "keysplit"): (1, 2, 512, 0), ("full", "4wave"): (1, 80, 512, 0),
          ("full", "8wave"): (2, 264, 512, 0),
          ("causal", "keysplit"): (1, 2, 512, 0), ("causal", "4wave"): (1, 80, 512, 0),
          ("causal", "8wave"): (2, 264, 512, 0),
          ("window", "4wave"): (1, 2, 1024, 300), ("window", "8wave"): (1, 64, 4096, 2500)}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,shape", sorted(SHAPES), ids=[f"{m}-{s}" for m, s in sorted(SHAPES)])
def test_fwd_rescale_with_growing_maximum(shape, mask, d, dtype):
    B, H, N, window = SHAPES[(mask, shape)]
    causal = mask != "full"
    seed = 9200 + d + 3 * (mask == "causal") + 5 * (mask == "window") + 7 * (shape == "8wave") + \
        11 * (shape == "keysplit")
    announce(f"fwd rescale {shape} {mask} B{B} H{H} N{N} d{d} window={window} {dtype} seed={seed}")
    q, k, v = ramp_inputs(B, H, N, d, dtype, seed)
    scale = d ** -0.5
    # premise: the running maximum outgrows the slack after the first tile, many times
    if window:
        def kbase(i):  # first tile the kernel loads for the row's block (block start - window)
            br = 128 if shape == "4wave" else 256
            return (max(0, (i // br) * br - window + 1) // TILE) * TILE
    else:
        def kbase(i):
            return 0
    events = count_rescales(q[0, 0], k[0, 0], scale, causal, window, kbase)
    assert events >= N // 4, f"inputs trigger only {events} rescales after the first tile"
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal, window)
    o_h, lse_h = host64(o), host64(lse)
    heads = [(0, 0), (B - 1, H - 1)] + ([(B - 1, H // 2)] if H > 2 else [])
    for b, h in heads:
        o_ref, lse_ref = oracle.attn_fwd(q[b, h], k[b, h], v[b, h], scale, causal, window=window)
        check_max_abs(o_h[b, h], o_ref, dtype, f"O head ({b},{h})")
        check_max_abs(lse_h[b, h], lse_ref, dtype, f"lse head ({b},{h})")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_with_growing_maximum(causal, dtype):
    """The backward rebuilds P from lse; on the same steep inputs its gradients must still
    match the oracle (whole tensor and every 32-row block)."""
    from tests.parity_util import check_rel_norm, check_rel_norm_blocks
    B, H, N, d = 1, 2, 512, 128
    seed = 9300 + (1 if causal else 0)
    announce(f"bwd on ramp inputs B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v = ramp_inputs(B, H, N, d, dtype, seed)
    do = attention_inputs(B, H, N, d, dtype, seed + 50, "cpu")[0]
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.attention_fwd(qd, kd, vd, scale, causal)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale, causal)
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.attn_bwd(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_rel_norm(host64(g[0, h]), r, dtype, f"{name} head {h}")
            check_rel_norm_blocks(host64(g[0, h]), r, dtype, f"{name} head {h}")
