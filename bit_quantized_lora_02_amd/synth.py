"""Seeded synthetic inputs for the NF4 + LoRA linear.

This module holds no arithmetic of the method: it only draws normal variates
with numpy's PCG64 and casts them to bfloat16 with torch's own (round to
nearest even) conversion.  Tests, the benchmark and the smoke check take their
inputs from here, so the GPU path and the CPU oracle see identical bits.

Recipe (one linear): ``SeedSequence(seed)`` spawns seven children, consumed in
this fixed order: W, outlier mask, outlier values, A, B, X, dY.
  W  ~ N(0, sigma_w) binary32 [n_out, n_in]; with ``outlier_frac`` > 0 each
       element is independently replaced, with that probability, by a
       N(0, outlier_sigma) draw;
  A  ~ N(0, 0.01) -> bf16 [r, n_in];   B ~ N(0, 0.01) -> bf16 [n_out, r];
  X  ~ N(0, 1)    -> bf16 [T, n_in];   dY ~ N(0, 1)   -> bf16 [T, n_out].
bf16 tensors are returned as their uint16 bit patterns.

The pages name no dataset or benchmark suite; roughly normal weights are what
they describe pretrained weights to look like, so these draws stand in for
pretrained weights and activations.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class LinearInputs:
    W: np.ndarray  # f32 [n_out, n_in]
    A: np.ndarray  # bf16 bits [r, n_in]
    B: np.ndarray  # bf16 bits [n_out, r]
    X: np.ndarray  # bf16 bits [T, n_in]
    dY: np.ndarray  # bf16 bits [T, n_out]
    alpha: float

    @property
    def shape(self):
        n_out, n_in = self.W.shape
        return dict(n_out=n_out, n_in=n_in, T=self.X.shape[0], r=self.A.shape[0])


def linear_inputs(n_out: int, n_in: int, T: int, r: int, alpha: float, seed: int = 0, sigma_w: float = 0.02,
                  outlier_frac: float = 0.0, outlier_sigma: float = 0.2, sigma_ab: float = 0.01,
                  sigma_x: float = 1.0, make_dy: bool = True) -> LinearInputs:
    ss = np.random.SeedSequence(seed)
    kw, km, kv, ka, kb, kx, kd = ss.spawn(7)
    W = np.random.Generator(np.random.PCG64(kw)).standard_normal((n_out, n_in), dtype=np.float32)
    W *= np.float32(sigma_w)
    if outlier_frac > 0.0:
        mask = np.random.Generator(np.random.PCG64(km)).random((n_out, n_in)) < outlier_frac
        vals = np.random.Generator(np.random.PCG64(kv)).standard_normal(int(mask.sum()), dtype=np.float32)
        W[mask] = vals * np.float32(outlier_sigma)
    g = lambda k, shape, s: to_bf16_bits(
        np.random.Generator(np.random.PCG64(k)).standard_normal(shape, dtype=np.float32) * np.float32(s))
    A = g(ka, (r, n_in), sigma_ab)
    B = g(kb, (n_out, r), sigma_ab)
    X = g(kx, (T, n_in), sigma_x)
    dY = g(kd, (T, n_out), 1.0) if make_dy else np.zeros((0, n_out), np.uint16)
    return LinearInputs(W=W, A=A, B=B, X=X, dY=dY, alpha=float(alpha))


# The five workloads.  Each entry: name -> list of linears (name, n_out, n_in) plus shared settings.
CONFIGS = {
    "cpu_256": dict(linears=[("proj", 256, 256)], T=16, r=8, alpha=16.0, outliers=0.0),
    "attn_4096": dict(linears=[("proj", 4096, 4096)], T=2048, r=16, alpha=32.0, outliers=0.0),
    "mlp_8b": dict(linears=[("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)], T=4096, r=64,
                   alpha=16.0, outliers=0.01),
    "small_token": dict(linears=[("sq", 8192, 8192), ("wide", 28672, 8192)], T=(1, 8, 32, 128), r=16, alpha=32.0,
                        outliers=0.0),
    "layer_70b": dict(linears=[("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
                               ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)], T=4096, r=64,
                      alpha=16.0, outliers=0.0),
}
