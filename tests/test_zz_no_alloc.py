"""GPU test of fa_decode_noalloc, the decode entry point that allocates nothing (its per-chunk
partials live in the library's static device scratch), against fa_decode_ex, the entry point
it is a variant of, on the same inputs through the C ABI.

Two calls in a row, the second with a smaller input (and another dtype, head dimension and
chunk count), so that the second runs on scratch the first left behind.  Each output must be
bitwise equal to fa_decode_ex's (the same kernels on the same inputs) and within the decode
tolerance of the float64 oracle; a call needing more scratch than the library holds must be
refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_max_abs, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (B, H, H_kv, Nkv, d, dtype, splits, seed): the first needs 16.1 MiB of scratch (the B64 H32
# d128 16-chunk decode's partials), the second 4.1 KiB.
CALLS = [(64, 32, 32, 1500, 128, torch.bfloat16, 16, 9101),
         (3, 4, 2, 300, 64, torch.float16, 5, 9102)]


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _one_call(B, H, Hkv, Nkv, d, dtype, splits, seed, heads_checked):
    announce(f"noalloc decode B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} {dtype} splits{splits} seed={seed}")
    need = fa.fa_decode_workspace_bytes(B, H, d, splits)
    assert need <= fa.FA_NOALLOC_SCRATCH_BYTES
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, DEV, Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    o_na = torch.full((B, H, 1, d), float("nan"), dtype=dtype, device=DEV)
    l_na = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_decode_noalloc(q, k, v, o_na, l_na, scale, splits)
    torch.cuda.synchronize()
    # the existing entry point on the same inputs, with a garbage-filled workspace of its own
    o_ex = torch.full_like(o_na, float("nan"))
    l_ex = torch.full_like(l_na, float("nan"))
    ws = fa.decode_workspace(k, splits, heads=H)
    ws.fill_(0xA5)
    fa.fa_decode_ex(q, k, v, o_ex, l_ex, scale, splits, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_na), _bits(o_ex)), "o differs from fa_decode_ex"
    assert torch.equal(_bits(l_na), _bits(l_ex)), "lse differs from fa_decode_ex"
    # and both against the float64 oracle on the checked heads
    for b, h in heads_checked:
        g = h // (H // Hkv)
        o_ref, l_ref = oracle.attn_decode(q[b, h].cpu(), k[b, g].cpu(), v[b, g].cpu(), scale)
        check_max_abs(host64(o_na[b, h, 0]), o_ref, dtype, f"o ({b},{h})")
        check_max_abs(host64(l_na[b, h]).reshape(()), np.asarray(l_ref), dtype, f"lse ({b},{h})")


def test_noalloc_decode_two_calls_second_smaller():
    B, H, Hkv, Nkv, d, dtype, splits, seed = CALLS[0]
    _one_call(B, H, Hkv, Nkv, d, dtype, splits, seed,
              [(0, 0), (0, 17), (31, 5), (63, 31)])
    B, H, Hkv, Nkv, d, dtype, splits, seed = CALLS[1]
    _one_call(B, H, Hkv, Nkv, d, dtype, splits, seed,
              [(b, h) for b in range(B) for h in range(H)])


def test_noalloc_decode_refuses_beyond_its_scratch():
    """64 x 64 heads x 32 chunks x 129 floats is more than the static scratch: FA_ERR_SCRATCH,
    and the outputs are not touched."""
    B, H, d, splits = 64, 64, 128, 32
    assert fa.fa_decode_workspace_bytes(B, H, d, splits) > fa.FA_NOALLOC_SCRATCH_BYTES
    announce(f"noalloc decode over the scratch limit B{B} H{H} d{d} splits{splits}")
    q, k, v = attention_inputs(B, H, 1, d, torch.bfloat16, 9103, DEV, Nkv=1)
    o = torch.full((B, H, 1, d), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError) as ei:
        fa.fa_decode_noalloc(q, k, v, o, lse, d ** -0.5, splits)
    assert ei.value.code == 9
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
