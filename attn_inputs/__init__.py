"""Seeded synthetic inputs for exact attention.

This module only draws random numbers and names workloads. It holds none of
the attention arithmetic, so that both the HIP path (through its tests and the
benchmark) and the CPU oracle can take their inputs from it without sharing
any of the method's code.

Every tensor is [B, H, N, d], contiguous, head dimension fastest, which is the
per-(batch, head) row layout that the pages index as Q[batch, head, rows, :]
(page "FlashAttention算子优化", §2 pseudocode; page "Attention 算子优化:从物化
N×N 矩阵到 FlashAttention 与 PagedAttention", §一).

Values are i.i.d. standard normal, which is the distribution the AIInfra
FlashAttention note (dpshk.com, §3.1) prescribes for the random-comparison
layer of its verification matrix. For 16-bit workloads the fp32 draws are
rounded to bfloat16 with round-to-nearest-even (torch's ``.to(bfloat16)``);
the very same bits are what the GPU path and the oracle both consume.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_inputs_device", "draw_seqlens",
           "workload", "fp8_cache", "fp8_head"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named synthetic workload.

    ``seqlen_range`` (inclusive) switches on a padded variable-length batch:
    one length per sequence, drawn uniformly from the range after the tensors.
    ``with_grad`` also draws the upstream gradient dO. ``H_kv`` (default H)
    gives K and V fewer heads than Q (grouped- or multi-query attention).
    ``Nq`` (default N) makes a decode workload: Q holds the last Nq positions
    of each sequence and K, V its N cached positions.
    """

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32", "bf16" or "f16"
    causal: bool
    seed: int
    seqlen_range: Optional[tuple[int, int]] = None
    with_grad: bool = False
    description: str = ""
    H_kv: Optional[int] = None
    Nq: Optional[int] = None
    kv_fp8: bool = False  # K/V stored as an FP8 cache (see fp8_cache)

    @property
    def kv_heads(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]


# The five workloads of this project: shapes, masks and precisions.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f32_n256_d64", 1, 1, 256, 64, "f32", False, 1001,
                 description="single head, non-causal, fp32, N=256, d=64"),
        Workload("mha_bf16_b4_h16_n2048_d64", 4, 16, 2048, 64, "bf16", False, 1002,
                 description="batched MHA forward, non-causal, bf16, B=4 H=16 N=2048 d=64"),
        Workload("causal_bf16_b2_h32_n4096_d128", 2, 32, 4096, 128, "bf16", True, 1003,
                 description="batched MHA forward, causal, bf16, B=2 H=32 N=4096 d=128"),
        Workload("varlen_bf16_b8_h16_n2048_d128", 8, 16, 2048, 128, "bf16", False, 1004,
                 seqlen_range=(512, 2048),
                 description="padded variable-length batch, key-padding mask, bf16, "
                             "8 sequences of length U{512..2048} padded to 2048, H=16 d=128"),
        Workload("causal_fwdbwd_bf16_b2_h16_n8192_d128", 2, 16, 8192, 128, "bf16", True, 1005,
                 with_grad=True,
                 description="forward + recompute backward, causal, bf16, B=2 H=16 N=8192 d=128"),
        Workload("causal_f16_b2_h32_n4096_d128", 2, 32, 4096, 128, "f16", True, 1007,
                 with_grad=True,
                 description="the causal B=2 H=32 N=4096 d=128 shape with fp16 inputs, fwd+bwd"),
        Workload("decode_bf16_b8_h64_hkv8_nq1_nk8192_d128", 8, 64, 8192, 128, "bf16", True, 1008,
                 H_kv=8, Nq=1,
                 description="decode: one new token per sequence, 64 query heads over 8 K/V "
                             "heads (the pages' 64:8 example), 8192 cached positions, bf16"),
        Workload("decode_bf16_b8_h64_hkv8_nq8_nk8192_d128", 8, 64, 8192, 128, "bf16", True, 1009,
                 H_kv=8, Nq=8, seqlen_range=(4096, 8192),
                 description="decode of 8 new tokens per sequence (causal among themselves) "
                             "over 4096..8192 cached positions, 64 query heads over 8 K/V heads"),
        Workload("decode_fp8kv_bf16_b8_h64_hkv8_nq1_nk8192_d128", 8, 64, 8192, 128, "bf16", True,
                 1010, H_kv=8, Nq=1, kv_fp8=True,
                 description="decode of one new token over an FP8 (E4M3, per-token scale) K/V "
                             "cache of 8192 positions, 64 query heads over 8 K/V heads"),
        Workload("gqa_causal_bf16_b2_h32_hkv8_n4096_d128", 2, 32, 4096, 128, "bf16", True, 1006,
                 with_grad=True, H_kv=8,
                 description="grouped-query attention, 32 query heads over 8 K/V heads (the "
                             "8:1 grouping of the pages' example), causal, bf16, fwd+bwd"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def draw_seqlens(gen: torch.Generator, B: int, lo: int, hi: int) -> torch.Tensor:
    """Per-sequence lengths, int32 uniform on the inclusive range [lo, hi]."""
    return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)


def make_inputs(B: int, H: int, N: int, d: int, dtype: torch.dtype = torch.bfloat16,
                seed: int = 0, with_grad: bool = False,
                seqlen_range: Optional[tuple[int, int]] = None,
                std: float = 1.0, H_kv: Optional[int] = None, Nq: Optional[int] = None) -> dict:
    """Draw Q, K, V (and dO, then seqlens) on the CPU from one seeded generator.

    The draw order is fixed (Q, K, V, dO, seqlens) so a workload is the same
    bits on every machine. K and V have H_kv heads (default H); Q (and dO)
    have Nq rows (default N). Returns CPU tensors in ``dtype``; ``seqlens`` is
    an int32 [B] tensor or None.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    kv_heads = H if H_kv is None else H_kv

    q_rows = N if Nq is None else Nq

    def draw(heads: int, rows: int = N) -> torch.Tensor:
        x = torch.randn((B, heads, rows, d), generator=gen, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        return x.to(dtype).contiguous()

    out = {"q": draw(H, q_rows), "k": draw(kv_heads), "v": draw(kv_heads)}
    out["do"] = draw(H, q_rows) if with_grad else None
    out["seqlens"] = (draw_seqlens(gen, B, *seqlen_range)
                      if seqlen_range is not None else None)
    return out


def make_inputs_device(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
                       device, H_kv: Optional[int] = None, Nq: Optional[int] = None,
                       with_grad: bool = False) -> dict:
    """Seeded N(0, 1) Q, K, V (and dO) drawn on ``device`` by a generator of that
    device, one batch entry at a time, for tensors too large to draw on the host
    in reasonable time (more than 2^31 elements). Same draw order and shapes as
    make_inputs; the values are the device generator's, not make_inputs'."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    kv_heads = H if H_kv is None else H_kv
    q_rows = N if Nq is None else Nq

    def draw(heads: int, rows: int) -> torch.Tensor:
        out = torch.empty((B, heads, rows, d), dtype=dtype, device=device)
        for b in range(B):
            out[b] = torch.randn((heads, rows, d), generator=gen, dtype=torch.float32,
                                 device=device).to(dtype)
        return out

    out = {"q": draw(H, q_rows), "k": draw(kv_heads, N), "v": draw(kv_heads, N)}
    out["do"] = draw(H, q_rows) if with_grad else None
    out["seqlens"] = None
    return out


def fp8_cache(x: torch.Tensor):
    """Store a K or V tensor [..., Nk, d] as an FP8 cache: one fp32 scale per
    token (row), amax / 448 (448 is E4M3's largest finite value), and the row
    divided by it rounded to E4M3 by torch's conversion. Returns (uint8 bytes,
    fp32 scales [..., Nk]). Rows of zeros get scale 1. This builds the inputs
    that both the HIP path and the oracle read; neither recomputes it."""
    xf = x.float()
    amax = xf.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q8 = (xf / scale[..., None]).to(torch.float8_e4m3fn)
    return q8.view(torch.uint8).contiguous(), scale.contiguous()


def fp8_head(x: torch.Tensor, valid_len=None):
    """Store a tensor [B, H, N, d] as FP8 with one fp32 scale per (batch, head):
    amax over the head's valid rows / 448, the head divided by it and rounded
    to E4M3 by torch's conversion. valid_len (int32 [B] or None) limits the
    amax to rows < L_b; rows at or past it are quantised like the others (a
    caller that wants them poisoned overwrites them). Returns (uint8 bytes,
    fp32 scales [B, H]). Heads of zeros get scale 1."""
    xf = x.float()
    if valid_len is not None:
        rows = torch.arange(x.shape[2])[None, :] < valid_len.to(torch.int64)[:, None]
        xf_valid = xf * rows[:, None, :, None]
    else:
        xf_valid = xf
    amax = xf_valid.abs().amax(dim=(-2, -1))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q8 = (xf / scale[..., None, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q8.view(torch.uint8).contiguous(), scale.contiguous()


def make_workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, w.with_grad, w.seqlen_range,
                       H_kv=w.H_kv, Nq=w.Nq)
