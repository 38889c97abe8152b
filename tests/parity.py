"""Shared tolerances and comparison metrics for the GPU parity tests.

Metrics follow the AIInfra FlashAttention note (dpshk.com, §3.1): max absolute
error, max relative error, cosine similarity and the NaN/Inf count are all
recorded; the pass/fail bar is max absolute error for outputs and relative
Frobenius error for gradients:
  O:   fp32 inputs <= 1e-5, bf16 inputs <= 2e-2 (oracle fed the same bf16 values),
       fp16 inputs <= 2.5e-3 (the bf16 bar scaled by fp16's 2^-3 smaller unit
       roundoff: 11 vs 8 significand bits; O's error comes from rounding P and O)
  LSE: fp32 <= 1e-5, bf16 and fp16 <= 1e-3 (the softmax statistics are kept in
       fp32; LSE sits before any 16-bit rounding, so its error is that of fp32
       score accumulation)
  dQ, dK, dV: ||g - g_ref||_F / ||g_ref||_F <= 5e-2 per tensor for bf16, 1e-2
       for fp16 (the bf16 bar scaled by 2^-3, rounded up). Where the oracle's
       gradient is exactly zero (a single visible key: dS = P o (dP - D) with
       dP = D), the relative error is undefined and the bar is max|g| <= 1e-5,
       the size of the fp32 rounding left in dP - D.
"""
from __future__ import annotations

import numpy as np
import torch

O_TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2.5e-3}
LSE_TOL = {"f32": 1e-5, "bf16": 1e-3, "f16": 1e-3}
GRAD_REL_FRO = 5e-2
GRAD_TOL = {"bf16": GRAD_REL_FRO, "f16": 1e-2}
GRAD_ZERO_ABS = 1e-5


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[t.dtype]


def to_np(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def metrics(got, ref) -> dict:
    g, r = to_np(got), to_np(ref)
    fin = np.isfinite(r)
    bad = int(np.sum(~np.isfinite(g[fin])))
    diff = np.abs(g[fin] - r[fin]) if fin.any() else np.zeros(1)
    denom = np.maximum(np.abs(r[fin]), 1e-6) if fin.any() else np.ones(1)
    gv, rv = g[fin].ravel(), r[fin].ravel()
    nrm = np.linalg.norm(gv) * np.linalg.norm(rv)
    return {"max_abs": float(diff.max()), "max_rel": float((diff / denom).max()),
            "cos": float(gv @ rv / nrm) if nrm > 0 else 1.0, "nonfinite": bad,
            "inf_mismatch": int(np.sum(np.isfinite(g) != fin))}


def assert_close(got, ref, tol: float, what: str) -> dict:
    m = metrics(got, ref)
    assert m["nonfinite"] == 0, f"{what}: {m['nonfinite']} NaN/Inf where the oracle is finite ({m})"
    assert m["inf_mismatch"] == 0, f"{what}: finiteness pattern differs from the oracle ({m})"
    assert m["max_abs"] <= tol, f"{what}: max abs err {m['max_abs']:.3e} > {tol:.1e} ({m})"
    return m


def rel_fro(got, ref) -> float:
    g, r = to_np(got), to_np(ref)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
