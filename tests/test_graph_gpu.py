"""HIP graph capture of the entry points (GPU).

fa_fwd, fa_bwd and fa_decode_noalloc are recorded into one graph with torch.cuda.graph and the
graph is replayed several times.  Between replays the program does its own eager work (every
output is refilled with NaN by torch) and synchronises.  Every replay must rewrite every output
and reproduce the eager results bitwise.  fa_decode_noalloc is the decode entry point for callers
that cannot allocate inside a capture: it takes no workspace (its per-chunk partials live in the
library's static scratch, whose address is looked up on the first, eager, call).  The library
records no memset: every kernel writes what the next one reads.
"""
import pytest
import torch

import exact_io_aware_31_amd as fa
from synth_inputs import attention_inputs
from tests.parity_util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_graph_replays_equal_eager(dtype):
    B, H, N, d = 2, 4, 1000, 128
    Bd, Hd, Hkv, Nkv, splits = 3, 8, 2, 3000, 7
    seed = 9500 + (dtype == torch.float16)
    announce(f"graph capture fwd/bwd B{B} H{H} N{N} d{d}, decode_noalloc B{Bd} H{Hd} Hkv{Hkv} "
             f"Nkv{Nkv} splits={splits} {dtype} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, DEV, with_dout=True)
    qd, kd, vd = attention_inputs(Bd, Hd, 1, d, dtype, seed + 1, DEV, Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    ws = fa.bwd_workspace(q)
    od = torch.empty_like(qd)
    lsed = torch.empty((Bd, Hd), dtype=torch.float32, device=DEV)
    outs = (o, lse, dq, dk, dv, od, lsed)

    def run():
        fa.fa_fwd(q, k, v, o, lse, scale, True)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, True)
        fa.fa_decode_noalloc(qd, kd, vd, od, lsed, scale, splits)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    for t in ref:
        assert bool(torch.isfinite(t.float()).all())

    # warm-up on a side stream, then capture (torch hands the capture stream to the binding)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("O", "lse", "dQ", "dK", "dV", "decode O", "decode lse"), outs, ref):
            assert torch.equal(_bits(t), _bits(r)), f"replay {rep}: {name} differs from eager"
    del graph
