"""Seeded synthetic inputs for the fused all-reduce-sum (+ residual + RMSNorm) workloads.

This module is the only code that both the oracle-side tests and the HIP-side tests/benchmark
use.  It generates inputs and nothing else: it holds none of the method's arithmetic.

Every tensor is drawn on the host from its own ``torch.Generator`` seeded with
``seed * 1009 + tensor_id`` (tensor_id = r for partial r, W for the residual, W + 1 for gamma),
in binary32, then rounded to the storage type with torch's round-to-nearest-even cast.
``N(mu, sigma)`` takes sigma as the standard deviation.

Workloads (shapes of the serving activations the pages tune the fused all-reduce for):
  tiny            W=2  M=4      H=256   bf16  partials N(0,1), residual N(0,1), gamma U(0.5,1.5),
                  eps 1e-6, residual+RMSNorm
  llama3_decode   W=2  M=128    H=4096  bf16  partials N(0,0.02), residual N(0,1),
                  gamma U(0.5,1.5), eps 1e-5, residual+RMSNorm  (Llama-3 concurrency-128 TP2
                  decode step of the flashinfer pull request "update allreduce to match trtllm")
  wide_hidden     W=8  M in {1,8,32,64,128,512,2048}  H=7168  bf16  partials N(0,0.05),
                  residual N(0,1), gamma U(0.8,1.2), eps 1e-6, both patterns  (the TP8 hidden-7168
                  M=1..2048 range of the tokenspeed pull request)
  large_sum       W=4  M=5120   H=8192  bf16  partials U(-1,1), plain sum  (80 MiB per rank, the
                  TP4 edge payload of the vLLM pull request's performance table)
  fp16_many_rank  W=16 M=512    H=8192  fp16  partials N(0,0.1) with 1% of elements replaced by
                  +-50 (fair sign), residual N(0,1), gamma U(0.5,1.5), eps 1e-6,
                  residual+RMSNorm  (the TP16 8 MiB payload of the same table)
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import torch

TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    W: int
    H: int
    Ms: Tuple[int, ...]
    dtype: str
    patterns: Tuple[str, ...]          # "sum" (kAllReduce) and/or "rms" (kARResidualRMSNorm)
    partial: Tuple                     # ("normal", mu, sigma) | ("uniform", lo, hi)
    residual: Optional[Tuple] = None
    gamma: Optional[Tuple] = None
    eps: Optional[float] = None
    outlier_frac: float = 0.0          # fraction of partial elements replaced by +-outlier_mag
    outlier_mag: float = 0.0
    seed: int = 20261202


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", W=2, H=256, Ms=(4,), dtype="bf16", patterns=("rms",),
                 partial=("normal", 0.0, 1.0), residual=("normal", 0.0, 1.0),
                 gamma=("uniform", 0.5, 1.5), eps=1e-6, seed=20261202),
        Workload("llama3_decode", W=2, H=4096, Ms=(128,), dtype="bf16", patterns=("rms",),
                 partial=("normal", 0.0, 0.02), residual=("normal", 0.0, 1.0),
                 gamma=("uniform", 0.5, 1.5), eps=1e-5, seed=20261203),
        Workload("wide_hidden", W=8, H=7168, Ms=(1, 8, 32, 64, 128, 512, 2048), dtype="bf16",
                 patterns=("sum", "rms"), partial=("normal", 0.0, 0.05),
                 residual=("normal", 0.0, 1.0), gamma=("uniform", 0.8, 1.2), eps=1e-6,
                 seed=20261204),
        Workload("large_sum", W=4, H=8192, Ms=(5120,), dtype="bf16", patterns=("sum",),
                 partial=("uniform", -1.0, 1.0), seed=20261205),
        Workload("fp16_many_rank", W=16, H=8192, Ms=(512,), dtype="fp16", patterns=("rms",),
                 partial=("normal", 0.0, 0.1), residual=("normal", 0.0, 1.0),
                 gamma=("uniform", 0.5, 1.5), eps=1e-6, outlier_frac=0.01, outlier_mag=50.0,
                 seed=20261206),
    ]
}


def _gen(seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1009 + tensor_id)
    return g


def draw(dist: Tuple, shape, g: torch.Generator) -> torch.Tensor:
    """Draw a binary32 tensor from ("normal", mu, sigma) or ("uniform", lo, hi)."""
    kind = dist[0]
    if kind == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32) * dist[2] + dist[1]
    if kind == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) * (dist[2] - dist[1]) + dist[1]
    raise ValueError("unknown distribution %r" % (kind,))


def partial(wl: Workload, r: int, M: int, seed: Optional[int] = None) -> torch.Tensor:
    """Partial r of workload ``wl`` at M tokens, as a CPU tensor of the storage type."""
    s = wl.seed if seed is None else seed
    g = _gen(s, r)
    x = draw(wl.partial, (M, wl.H), g)
    if wl.outlier_frac > 0.0:
        hit = torch.rand((M, wl.H), generator=g) < wl.outlier_frac
        sign = torch.where(torch.rand((M, wl.H), generator=g) < 0.5, -1.0, 1.0)
        x = torch.where(hit, sign * wl.outlier_mag, x)
    return x.to(TORCH_DTYPES[wl.dtype])


def residual(wl: Workload, M: int, seed: Optional[int] = None) -> torch.Tensor:
    s = wl.seed if seed is None else seed
    return draw(wl.residual, (M, wl.H), _gen(s, wl.W)).to(TORCH_DTYPES[wl.dtype])


def gamma(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    s = wl.seed if seed is None else seed
    return draw(wl.gamma, (wl.H,), _gen(s, wl.W + 1))


def inputs(wl: Workload, M: int, seed: Optional[int] = None):
    """(partials, residual, gamma) on the host; residual/gamma are None for a plain-sum workload."""
    parts: List[torch.Tensor] = [partial(wl, r, M, seed) for r in range(wl.W)]
    if "rms" not in wl.patterns:
        return parts, None, None
    return parts, residual(wl, M, seed), gamma(wl, seed)


def custom(W: int, M: int, H: int, dtype: str, seed: int, dist=("normal", 0.0, 1.0),
           with_norm: bool = True, outlier_frac: float = 0.0, outlier_mag: float = 0.0):
    """Inputs of an arbitrary shape (edge-case tests): N(0,1)-like partials and residual,
    gamma U(0.5, 1.5)."""
    wl = Workload("custom", W=W, H=H, Ms=(M,), dtype=dtype,
                  patterns=("sum", "rms") if with_norm else ("sum",), partial=dist,
                  residual=("normal", 0.0, 1.0), gamma=("uniform", 0.5, 1.5), eps=1e-6,
                  outlier_frac=outlier_frac, outlier_mag=outlier_mag, seed=seed)
    return inputs(wl, M)


def storage_numpy(t: torch.Tensor):
    """Host tensor -> numpy storage array (uint16 bit patterns for 16-bit types)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view("uint16")
