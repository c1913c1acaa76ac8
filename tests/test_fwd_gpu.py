"""GPU parity of fa_fwd against the float64 oracle (called through the C ABI)."""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import FWD_2K, FWD_8K, TINY_FWD, attention_inputs
from tests.parity_util import announce, check_max_abs, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_fwd(q, k, v, scale, causal):
    """Outputs start as NaN so an element the kernel never writes fails the check."""
    B, H, N, d = q.shape
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd(q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1, 17, 64, 127, 128, 129, 300, 1000])
def test_fwd_sweep(N, causal, d, dtype):
    B, H = 2, 3
    seed = 7000 + N + 13 * d + (1 if causal else 0)
    announce(f"fwd sweep B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu")
    scale = d ** -0.5
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    check_max_abs(host64(o), o_ref, dtype, "O")
    check_max_abs(host64(lse), lse_ref, dtype, "lse")


def test_fwd_tiny_workload():
    w = TINY_FWD
    announce(f"fwd {w.name} seed={w.seed}")
    q, k, v = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, "cpu")
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.scale, w.causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.scale, w.causal)
    check_max_abs(host64(o), o_ref, w.dtype, "O")
    check_max_abs(host64(lse), lse_ref, w.dtype, "lse")


def sampled_rows(N, n_random, rng):
    rows = set(range(0, min(N, 96)))             # early causal rows: few keys, large |O|
    rows.update(range(max(0, N - 32), N))        # last rows: all keys
    rows.update(rng.choice(N, size=min(N, n_random), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("w", [FWD_2K, FWD_8K], ids=lambda w: w.name)
def test_fwd_full_size_workloads(w):
    """Full-size launch; the oracle checks whole heads and sampled rows of every head."""
    announce(f"fwd {w.name} seed={w.seed} (inputs drawn on the host)")
    q, k, v = attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, "cpu", q_mult=w.q_mult)
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.scale, w.causal)
    o_h, lse_h = host64(o), host64(lse)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h)), "unwritten outputs"
    # causal row 0 sees only key 0, so its output is exactly V[..., 0, :]
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    rng = np.random.default_rng(w.seed)
    B, H = w.B, w.H
    full_heads = [(0, 0), (B - 1, H - 1)]
    for b, h in full_heads:
        o_ref, lse_ref = oracle.attn_fwd(q[b, h], k[b, h], v[b, h], w.scale, w.causal)
        check_max_abs(o_h[b, h], o_ref, w.dtype, f"O head ({b},{h})")
        check_max_abs(lse_h[b, h], lse_ref, w.dtype, f"lse head ({b},{h})")
    for b in range(B):
        for h in range(H):
            if (b, h) in full_heads:
                continue
            rows = sampled_rows(w.N, 64, rng)
            o_ref, lse_ref = oracle.attn_fwd(q[b, h, rows], k[b, h], v[b, h], w.scale, w.causal,
                                             qpos=rows)
            check_max_abs(o_h[b, h, rows], o_ref, w.dtype, f"O head ({b},{h}) rows")
            check_max_abs(lse_h[b, h, rows], lse_ref, w.dtype, f"lse head ({b},{h}) rows")


def test_fwd_deterministic():
    w = FWD_2K
    announce("fwd determinism (two runs, bitwise)")
    q, k, v = (t.to(DEV) for t in attention_inputs(2, 4, 1000, 128, torch.bfloat16, 99, "cpu"))
    o1, l1 = run_fwd(q, k, v, w.scale, True)
    o2, l2 = run_fwd(q, k, v, w.scale, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("H", [64, 65], ids=["4wave", "8wave"])
def test_fwd_both_workgroup_shapes(H, causal, d, dtype):
    """B4 N1024: 64 heads give 1024 blocks of 256 rows, the most that blocks of N <= 2048 run
    as four-wave workgroups (two per CU); 65 heads give 1040 and run eight-wave ones.  Whole
    heads spread over the grid against the oracle."""
    B, N = 4, 1024
    seed = 7300 + H + d + (1 if causal else 0)
    announce(f"fwd shapes B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu")
    scale = d ** -0.5
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal)
    o_h, lse_h = host64(o), host64(lse)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h)), "unwritten outputs"
    for b, h in [(0, 0), (1, H // 2), (3, H - 1)]:
        o_ref, lse_ref = oracle.attn_fwd(q[b, h], k[b, h], v[b, h], scale, causal)
        check_max_abs(o_h[b, h], o_ref, dtype, f"O head ({b},{h})")
        check_max_abs(lse_h[b, h], lse_ref, dtype, f"lse head ({b},{h})")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64)],
                         ids=["bf16-d128", "f16-d64"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("H,N", [(4, 4096), (4, 4097), (2, 4000), (8, 4096), (8, 4097)],
                         ids=["keysplit-256", "4wave-260", "keysplit-odd-tiles", "512",
                              "520"])
def test_fwd_key_split_boundary(H, N, causal, d, dtype):
    """Grids of at most 256 blocks of 64 rows (512 at d = 64) run four-wave workgroups whose
    two pairs of waves split each step's keys and merge at the end: B1 H4 N4096 is 256 such
    blocks, N4097 is 260 and runs the plain four-wave shape; N4000 leaves an odd number of key
    tiles, so the last step's second tile starts past the end; B1 H8 N4096 (512 blocks) splits
    at d = 64 only, N4097 (520) at neither.  Every head against the oracle."""
    B = 1
    seed = 7400 + H + N + d + (1 if causal else 0)
    announce(f"fwd key split B{B} H{H} N{N} d{d} causal={causal} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, N, d, dtype, seed, "cpu")
    scale = d ** -0.5
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal)
    o_h, lse_h = host64(o), host64(lse)
    for h in range(H):
        o_ref, lse_ref = oracle.attn_fwd(q[0, h], k[0, h], v[0, h], scale, causal)
        check_max_abs(o_h[0, h], o_ref, dtype, f"O head {h}")
        check_max_abs(lse_h[0, h], lse_ref, dtype, f"lse head {h}")
