"""The backward's second stream (GPU).

On grids of at most 512 blocks of 128 keys, fa_bwd runs its dQ kernel on a stream of the
library's, forked from the caller's stream after the row-term kernel and joined back into it
after the dQ kernel.  These tests check the ordering that promises:
  * work queued on the caller's stream after the call sees the finished gradients;
  * calls from two host threads, on two streams of one device, each pair their own fork and
    join (the outputs of every call equal a lone call's, bitwise);
  * a backward captured into a graph before the library has made its second stream (a fresh
    process) runs on the capturing stream alone, and its replays equal the eager result;
  * grouped key/value heads, which take the second stream at any grid size, past 512 blocks
    (against the oracle on sampled groups).
The kernels are the same on one or two streams, so every comparison is bitwise.
"""
import os
import subprocess
import sys
import threading

import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import attention_inputs
from tests.parity_util import announce, check_rel_norm, check_rel_norm_blocks, host64

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bits(t):
    return t.view(torch.int16)


def _forward(q, k, v, scale, causal):
    o, lse = fa.attention_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    return o, lse


def test_work_after_the_call_sees_the_gradients():
    """B1 H4 N8192 causal (256 key blocks): the dQ kernel runs ~0.3 ms on the second stream.
    Copies queued on the caller's stream right after the call must hold the final gradients."""
    B, H, N, d, dtype, seed = 1, 4, 8192, 128, torch.bfloat16, 9990
    announce(f"bwd join B{B} H{H} N{N} d{d} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, DEV, with_dout=True)
    scale = d ** -0.5
    o, lse = _forward(q, k, v, scale, True)
    ws = fa.bwd_workspace(q)
    ref = fa.attention_bwd(q, k, v, o, lse, do, scale, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for rep in range(3):
            dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
            fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, True)
            copies = [t.clone() for t in (dq, dk, dv)]  # queued on s, no synchronisation
            s.synchronize()
            for name, c, r in zip(("dQ", "dK", "dV"), copies, ref):
                assert torch.equal(_bits(c), _bits(r)), f"call {rep}: {name} copied before done"


def test_two_host_threads_on_two_streams():
    """Two threads call fa_bwd on their own streams at once, 20 times each (B1 H8 N1024 causal,
    64 key blocks); every call's gradients equal a lone call's."""
    B, H, N, d, dtype, seed = 1, 8, 1024, 128, torch.bfloat16, 9991
    announce(f"bwd two threads B{B} H{H} N{N} d{d} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, DEV, with_dout=True)
    scale = d ** -0.5
    o, lse = _forward(q, k, v, scale, True)
    ref = fa.attention_bwd(q, k, v, o, lse, do, scale, True)
    torch.cuda.synchronize()
    failures = []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            ws = fa.bwd_workspace(q)
            outs = [torch.empty_like(q) for _ in range(3)]
            torch.cuda.synchronize()
            for rep in range(20):
                with torch.cuda.stream(s):
                    for t in outs:
                        t.fill_(float("nan"))
                    fa.fa_bwd(q, k, v, o, lse, do, *outs, ws, scale, True)
                s.synchronize()
                for name, t, r in zip(("dQ", "dK", "dV"), outs, ref):
                    if not torch.equal(_bits(t), _bits(r)):
                        failures.append(f"thread {tid} call {rep}: {name}")
        except Exception as e:  # reported below, with the thread
            failures.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not failures, failures[:5]


_FRESH_CAPTURE = r"""
import sys, torch
sys.path.insert(0, ROOT)
sys.path.insert(0, ROOT + "/tests")
import exact_io_aware_31_amd as fa
from synth_inputs import attention_inputs
B, H, N, d = 2, 4, 1000, 128
q, k, v, do = attention_inputs(B, H, N, d, torch.bfloat16, 9992, "cuda", with_dout=True)
scale = d ** -0.5
o, lse = fa.attention_fwd(q, k, v, scale, True)
ws = fa.bwd_workspace(q)
outs = [torch.empty_like(q) for _ in range(3)]
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # the first backward of this process
    fa.fa_bwd(q, k, v, o, lse, do, *outs, ws, scale, True)
torch.cuda.synchronize()
ref = fa.attention_bwd(q, k, v, o, lse, do, scale, True)  # eager: makes the second stream
torch.cuda.synchronize()
for rep in range(3):
    for t in outs:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for name, t, r in zip(("dQ", "dK", "dV"), outs, ref):
        assert torch.equal(t.view(torch.int16), r.view(torch.int16)), (rep, name)
print("fresh capture ok", flush=True)
"""


def test_capture_before_the_second_stream_exists():
    announce("bwd captured first in a fresh process B2 H4 N1000 d128 seed=9992")
    code = _FRESH_CAPTURE.replace("ROOT", repr(ROOT))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "fresh capture ok" in r.stdout, (r.stdout[-2000:],
                                                                  r.stderr[-2000:])


def test_grouped_heads_past_512_blocks():
    """B32 H4 H_kv2 N1152 causal: 576 blocks of 128 keys, grouped heads, so the dQ pass runs
    beside the dK/dV pass; sampled key/value groups against the oracle."""
    B, H, Hkv, N, d, dtype, seed = 32, 4, 2, 1152, 128, torch.bfloat16, 9993
    announce(f"bwd grouped two streams B{B} H{H} Hkv{Hkv} N{N} d{d} seed={seed}")
    q, k, v, do = attention_inputs(B, H, N, d, dtype, seed, "cpu", with_dout=True, Hkv=Hkv)
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.attention_fwd(qd, kd, vd, scale, True)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale, True)
    torch.cuda.synchronize()
    dq_h, dk_h, dv_h = host64(dq), host64(dk), host64(dv)
    g = H // Hkv
    for b, hk in [(0, 0), (17, 1), (B - 1, Hkv - 1)]:
        hs = slice(g * hk, g * hk + g)
        ref = oracle.attn_bwd(q[b, hs], k[b, hk:hk + 1], v[b, hk:hk + 1], do[b, hs], scale, True)
        for name, gt, r in (("dQ", dq_h[b, hs], ref[0]), ("dK", dk_h[b, hk:hk + 1], ref[1]),
                            ("dV", dv_h[b, hk:hk + 1], ref[2])):
            check_rel_norm(gt, r, dtype, f"{name} group ({b},{hk})")
            check_rel_norm_blocks(gt, r, dtype, f"{name} group ({b},{hk})")
