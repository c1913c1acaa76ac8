"""GPU parity of the grouped-head decode (several query heads per key/value head) against the
float64 oracle, through the C ABI ("FlashAttention ontleed", § "Interactie met de KV-cache tijdens
inferentie": query heads that share one key/value head).

With H / H_kv >= 2 query heads per key/value head the chunk kernel runs the matrix-core path: one
workgroup takes G query heads (G the largest divisor of the group that is at most 16, so groups
above 16 take several workgroups per key/value head), four waves each take every fourth 32-key tile
of the chunk, and the waves merge by the online-softmax rule at the end.  The cases cover:
  * group sizes 2 .. 48, including ones that are not powers of two (3, 5, 6, 12), a prime above
    16 (17: one head per workgroup) and multiples of 16 (32, 48: two and three workgroups per
    key/value head);
  * chunks of fewer than four tiles (waves with no tile), tiles cut by the chunk's end, and
    chunks that are not multiples of 32 keys;
  * a running maximum that grows by more than the kernel's rescale slack (2^8 in exp2 units)
    from tile to tile within each wave (Lensa ML explainer, Step 4: the running sum and output
    are rescaled when a later block holds a larger score);
  * the full-size grouped workload (B64 H32 H_kv 8, 16384 keys) and its ragged-history variant,
    on sampled heads.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_31_amd as fa
import oracle
from synth_inputs import GQA_DECODE_16K, attention_inputs, ragged_lengths
from tests.parity_util import announce, check_max_abs, host64, nan_like

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILE = 32          # keys per tile of the grouped kernel
WAVES = 4          # waves per workgroup, each taking every fourth tile
SLACK_LOG2 = 8.0   # rescale slack, in log2 units


def run_decode(q, k, v, scale, splits, kv_lens=None):
    B, H = q.shape[0], q.shape[1]
    o = nan_like(q)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    ws = fa.decode_workspace(k, splits, heads=H)
    ws.fill_(0xFF)
    if kv_lens is None:
        fa.fa_decode_ex(q, k, v, o, lse, scale, splits, ws)
    else:
        fa.fa_decode_varlen(q, k, v, kv_lens, o, lse, scale, splits, ws)
    torch.cuda.synchronize()
    return o, lse


def check_all(q, k, v, o, lse, scale, dtype, kv_lens=None):
    o_ref, lse_ref = oracle.attn_decode(q, k, v, scale, kv_lens=kv_lens)
    got_o, got_lse = host64(o)[:, :, 0], host64(lse)
    if kv_lens is None:
        check_max_abs(got_o, o_ref, dtype, "O")
        check_max_abs(got_lse, lse_ref, dtype, "lse")
        return
    for b, n in enumerate(kv_lens):
        if n == 0:
            assert not np.any(got_o[b]) and np.all(got_lse[b] == -np.inf)
            continue
        check_max_abs(got_o[b], o_ref[b], dtype, f"O seq {b} (len {n})")
        check_max_abs(got_lse[b], lse_ref[b], dtype, f"lse seq {b} (len {n})")


# (B, H, H_kv, Nkv, splits): group sizes 2 .. 48
GROUPS = [(2, 8, 4, 1000, 4), (1, 6, 2, 777, 3), (2, 10, 2, 300, 2), (1, 12, 2, 2049, 5),
          (1, 8, 1, 1500, 1), (1, 24, 2, 640, 7), (2, 16, 1, 999, 16), (1, 17, 1, 700, 2),
          (1, 32, 1, 1111, 3), (1, 48, 1, 513, 1)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,Nkv,splits", GROUPS,
                         ids=[f"group{h // kv}" for _, h, kv, _, _ in GROUPS])
def test_decode_group_sizes(B, H, Hkv, Nkv, splits, d, dtype):
    seed = 9600 + H + Hkv + d + Nkv
    announce(f"decode group B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} {dtype} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    o, lse = run_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, splits)
    check_all(q, k, v, o, lse, scale, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nkv,splits", [(1, 1), (5, 1), (31, 1), (32, 1), (33, 1), (65, 1),
                                        (97, 1), (127, 1), (128, 1), (129, 1), (100, 3),
                                        (300, 16), (4097, 16)])
def test_decode_group_short_and_ragged_chunks(Nkv, splits, d):
    """Chunks of fewer than four tiles leave some waves without a tile; chunk ends that are
    not multiples of 32 keys cut the last tile."""
    B, H, Hkv, dtype = 2, 8, 2, torch.bfloat16
    seed = 9650 + Nkv + splits + d
    announce(f"decode group chunks B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} seed={seed}")
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=Nkv, Hkv=Hkv)
    scale = d ** -0.5
    o, lse = run_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, splits)
    check_all(q, k, v, o, lse, scale, dtype)


def ramp_decode_inputs(B, H, Hkv, Nkv, d, dtype, seed, a=8.0, top=64.0):
    """N(0,1) inputs with q[..., 0] = a and k[..., j, 0] = top * j / Nkv (rounded to dtype), V
    halved: every head's scores rise steadily along the history, so the running maximum
    outgrows the slack tile after tile (V halved keeps |O| where a bf16 output's own rounding
    leaves room for the rounding of P, as in the forward's test on the same recipe)."""
    q, k, v = attention_inputs(B, H, 1, d, dtype, seed, "cpu", Nkv=Nkv, Hkv=Hkv)
    q[..., 0] = a
    k[..., 0] = (torch.arange(Nkv, dtype=torch.float32) * (top / Nkv)).to(dtype)
    v = (v.float() * 0.5).to(dtype)
    return q, k, v


def count_decode_rescales(q, k, scale, splits):
    """Rescales after each wave's first tile, in float64 log2 units, as the kernel walks its
    tiles: chunk c of ceil(Nkv / splits) keys, wave w takes tiles w, w + 4, ... of the chunk."""
    s = (q.double().numpy() @ k.double().numpy().T) * scale * np.log2(np.e)   # [nkv]
    nkv = s.shape[-1]
    chunk = -(-nkv // splits)
    events = 0
    for c0 in range(0, nkv, chunk):
        c1 = min(nkv, c0 + chunk)
        for w in range(WAVES):
            ref, first = -np.inf, True
            for t0 in range(c0 + TILE * w, c1, TILE * WAVES):
                m = s[t0:min(c1, t0 + TILE)].max()
                if m > ref + SLACK_LOG2:
                    events += 0 if first else 1
                    ref = m
                first = False
    return events


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv,splits", [(8, 2, 1), (16, 1, 3)], ids=["group4", "group16"])
def test_decode_group_rescale_with_growing_maximum(H, Hkv, splits, d, dtype):
    B, Nkv = 1, 2048
    seed = 9680 + H + d + splits
    announce(f"decode group rescale B{B} H{H} Hkv{Hkv} Nkv{Nkv} d{d} splits={splits} {dtype} "
             f"seed={seed}")
    q, k, v = ramp_decode_inputs(B, H, Hkv, Nkv, d, dtype, seed)
    scale = d ** -0.5
    # premise: within every wave the reference maximum is moved again after its first tile
    for h in (0, H - 1):
        events = count_decode_rescales(q[0, h, 0], k[0, h // (H // Hkv)], scale, splits)
        assert events >= 4 * splits, f"head {h}: only {events} rescales after the first tile"
    o, lse = run_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, splits)
    check_all(q, k, v, o, lse, scale, dtype)


def test_decode_group_ragged_rescale():
    """Ragged histories on the same steep inputs: each sequence's chunks end at its length."""
    B, H, Hkv, Nkv, d, dtype, splits = 4, 8, 2, 2048, 128, torch.bfloat16, 2
    lens = [2048, 1000, 33, 1537]
    seed = 9690
    announce(f"decode group ragged rescale B{B} H{H} Hkv{Hkv} Nkv{Nkv} lens={lens} seed={seed}")
    q, k, v = ramp_decode_inputs(B, H, Hkv, Nkv, d, dtype, seed)
    scale = d ** -0.5
    kv_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = run_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, splits, kv_lens)
    check_all(q, k, v, o, lse, scale, dtype, kv_lens=lens)


def _sampled_heads(w, rng):
    return [(0, 0), (w.B - 1, w.H - 1)] + [(int(b), int(rng.integers(w.H))) for b in
                                           rng.choice(w.B, size=24, replace=False)]


@pytest.mark.parametrize("ragged", [False, True], ids=["full", "ragged"])
def test_decode_group_full_size_workload(ragged):
    """B64 H32 H_kv 8, 16384 keys, 16 chunks (4.3 GB of K/V drawn on the GPU); the oracle checks
    sampled heads.  Ragged: seeded history lengths uniform in [1, 16384] per sequence."""
    w = GQA_DECODE_16K
    announce(f"decode {w.name}{' ragged' if ragged else ''} seed={w.seed} (inputs drawn on the GPU)")
    q, k, v = attention_inputs(w.B, w.H, 1, w.d, w.dtype, w.seed, DEV, Nkv=w.Nkv, Hkv=w.Hkv)
    lens = ragged_lengths(w.B, w.Nkv, w.seed) if ragged else None
    o, lse = run_decode(q, k, v, w.scale, w.splits,
                        lens.to(DEV) if ragged else None)
    o_h, lse_h = host64(o)[:, :, 0], host64(lse)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h)), "unwritten outputs"
    group = w.H // w.Hkv
    for b, h in _sampled_heads(w, np.random.default_rng(w.seed + ragged)):
        n = int(lens[b]) if ragged else w.Nkv
        o_ref, lse_ref = oracle.attn_decode(q[b, h].cpu(), k[b, h // group, :n].cpu(),
                                            v[b, h // group, :n].cpu(), w.scale)
        check_max_abs(o_h[b, h], o_ref, w.dtype, f"O head ({b},{h})")
        check_max_abs(np.array(lse_h[b, h]), np.array(lse_ref), w.dtype, f"lse head ({b},{h})")
    del k, v
    torch.cuda.empty_cache()


def test_attention_decode_with_history_lengths():
    """The binding's attention_decode(kv_lens=...) is fa_decode_varlen: bitwise the same output."""
    B, H, Hkv, Nkv, d, dtype, splits = 3, 8, 2, 500, 128, torch.bfloat16, 4
    announce(f"attention_decode kv_lens B{B} H{H} Hkv{Hkv} Nkv{Nkv} splits={splits}")
    q, k, v = (t.to(DEV) for t in attention_inputs(B, H, 1, d, dtype, 9695, "cpu", Nkv=Nkv,
                                                    Hkv=Hkv))
    kv_lens = torch.tensor([500, 0, 77], dtype=torch.int32, device=DEV)
    o1, l1 = fa.attention_decode(q, k, v, d ** -0.5, num_splits=splits, kv_lens=kv_lens)
    o2, l2 = run_decode(q, k, v, d ** -0.5, splits, kv_lens)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
