"""Seeded synthetic inputs for attention tests and benchmarks.

This module is the only code shared by the HIP path's tests/benchmark and the
float64 oracle.  It holds no attention arithmetic: it only draws i.i.d.
N(0, 1) values, optionally multiplies Q by an exact power of two, and rounds
to the storage dtype (round-to-nearest-even, torch's ``.to``).

Draw order for a workload is Q, K, V, dO, each as float32 ``randn`` from one
``torch.Generator`` seeded with the workload's seed, on the requested device.
The same seed on another device gives other (equally valid) values; the
oracle always receives the exact bits the GPU received, copied back.

Large tensors are drawn one batch row at a time (same generator stream, in
order) so the float32 staging buffer stays at one [H, N, d] slice.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd", "bwd" or "decode"
    B: int
    H: int
    N: int               # query length (fwd/bwd) -- 1 for decode
    d: int
    dtype: torch.dtype
    causal: bool
    seed: int
    q_mult: float = 1.0  # exact power-of-two factor applied to Q
    Nkv: int = 0         # key/value length for decode
    splits: int = 0      # history chunks per head for decode
    Hkv: int = 0         # key/value heads (0: as many as query heads)
    window: int = 0      # causal sliding window (0: none)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


# The five workloads the attention path is specified on.
TINY_FWD = Workload("tiny_fwd_b1h1n256d64_f16", "fwd", 1, 1, 256, 64, torch.float16, False, 1001,
                    note="non-causal, fp16")
FWD_2K = Workload("fwd_b4h16n2048d128_bf16_causal", "fwd", 4, 16, 2048, 128, torch.bfloat16,
                  True, 1002)
FWD_8K = Workload("fwd_b1h32n8192d128_bf16_causal_q2", "fwd", 1, 32, 8192, 128, torch.bfloat16,
                  True, 1003, q_mult=2.0, note="Q scaled x2 to sharpen softmax")
BWD_4K = Workload("bwd_b2h16n4096d128_bf16_causal", "bwd", 2, 16, 4096, 128, torch.bfloat16,
                  True, 1004)
DECODE_16K = Workload("decode_b64h32kv16384d128_bf16_s16", "decode", 64, 32, 1, 128,
                      torch.bfloat16, False, 1005, Nkv=16384, splits=16)

# Grouped key/value heads and a sliding window on the same shapes.
GQA_DECODE_16K = Workload("decode_b64h32kv8_kv16384d128_bf16_s16", "decode", 64, 32, 1, 128,
                          torch.bfloat16, False, 1006, Nkv=16384, splits=16, Hkv=8,
                          note="4 query heads per key/value head")
WINDOW_FWD_8K = Workload("fwd_b1h32n8192d128_bf16_window1024", "fwd", 1, 32, 8192, 128,
                         torch.bfloat16, True, 1007, window=1024,
                         note="causal sliding window of 1024 keys")

WORKLOADS = {w.name: w for w in (TINY_FWD, FWD_2K, FWD_8K, BWD_4K, DECODE_16K, GQA_DECODE_16K,
                                 WINDOW_FWD_8K)}


def _draw(gen: torch.Generator, shape, dtype, device, mult: float = 1.0) -> torch.Tensor:
    """float32 N(0,1) -> optional exact scaling -> round to dtype, batch row by row."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32, device=device)
        if mult != 1.0:
            x.mul_(mult)
        out[b].copy_(x)
        del x
    return out


def attention_inputs(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
                     device="cpu", q_mult: float = 1.0, with_dout: bool = False,
                     Nkv: Optional[int] = None, Hkv: Optional[int] = None):
    """Q [B,H,N,d], K and V [B,Hkv or H,Nkv or N,d] (and dO like Q) drawn in that order."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    nk = N if Nkv is None else Nkv
    hk = H if Hkv is None else Hkv
    q = _draw(gen, (B, H, N, d), dtype, device, q_mult)
    k = _draw(gen, (B, hk, nk, d), dtype, device)
    v = _draw(gen, (B, hk, nk, d), dtype, device)
    if not with_dout:
        return q, k, v
    do = _draw(gen, (B, H, N, d), dtype, device)
    return q, k, v, do


def ragged_lengths(B: int, Nkv: int, seed: int):
    """Seeded history lengths for a padded cache of B sequences, uniform in [1, Nkv]
    (int32, on the host)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.randint(1, Nkv + 1, (B,), generator=gen, dtype=torch.int32)


def workload_inputs(w: Workload, device="cpu"):
    """Inputs of a named workload (decode: q is [B,H,1,d])."""
    hkv = w.Hkv or None
    if w.kind == "decode":
        return attention_inputs(w.B, w.H, 1, w.d, w.dtype, w.seed, device, w.q_mult,
                                Nkv=w.Nkv, Hkv=hkv)
    return attention_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, device, w.q_mult,
                            with_dout=(w.kind == "bwd"), Hkv=hkv)
