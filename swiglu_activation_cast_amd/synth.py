"""Seeded synthetic inputs for the workloads (no part of the cast itself).

Shapes and value distributions of the workloads the pages measure ("Add
swiglu + MXFP8 fused CuTe DSL kernel", Performance: activations up to
131072 x 8192 per operand; "[mxfp8 moe training] update 3d quant colwise
scaling kernel ...", Performance: expert weights (E, 8192, 5120)).  The
pages do not give value distributions; the ones used here are stated per
workload.  Values are drawn as float32 normals with a seeded torch
generator on the target device, scaled, and rounded to bf16 (round to
nearest even).  Large tensors are drawn in row chunks so that memory stays
bounded; the chunking is part of the recipe, so a given (seed, shape,
device type) always gives the same bits.

This module is shared by the tests, the smoke check and the benchmark; it
holds no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

_CHUNK_ELEMS = 1 << 26  # elements drawn per generator call


def normal_bf16(shape, std: float, seed: int, device="cpu", gen: Optional[torch.Generator] = None) -> torch.Tensor:
    """bf16 tensor of N(0, std^2) values; rows drawn in fixed-size chunks."""
    device = torch.device(device)
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[s:e] = x.to(torch.bfloat16)
    return out


def add_outliers_(t: torch.Tensor, rate: float, factor: float, gen: torch.Generator) -> torch.Tensor:
    """Multiply a Bernoulli(rate) subset of elements by `factor`, in place."""
    mask = torch.rand(t.shape, generator=gen, device=t.device) < rate
    t[mask] = (t[mask].float() * factor).to(torch.bfloat16)
    return t


def zero_tiles_(tensors, tile: int, rate: float, gen: torch.Generator):
    """Zero the same randomly chosen aligned tile x tile squares in every tensor."""
    M, N = tensors[0].shape
    pick = torch.rand((M // tile, N // tile), generator=gen, device=tensors[0].device) < rate
    mask = pick.repeat_interleave(tile, 0).repeat_interleave(tile, 1)
    for t in tensors:
        t.masked_fill_(mask, 0)
    return tensors


@dataclass
class SwigluInputs:
    gate: torch.Tensor
    up: torch.Tensor
    dh: torch.Tensor
    w13: Optional[torch.Tensor] = None  # set when gate/up are halves of one [M, 2N] tensor


def swiglu_inputs(M: int, N: int, *, seed: int, std: float = 1.0, packed: bool = False,
                  outlier_rate: float = 0.0, outlier_factor: float = 100.0, zero_tile_rate: float = 0.0,
                  device="cpu") -> SwigluInputs:
    """gate, up and dh of shape [M, N].

    packed: gate and up are the halves of one [M, 2N] w13 tensor (drawn as a
    whole), as a fused w13 projection produces them.  Otherwise gate, up and
    dh are drawn one after another from the same generator.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w13 = None
    if packed:
        w13 = normal_bf16((M, 2 * N), std, seed, device, gen)
        gate, up = w13[:, :N], w13[:, N:]
    else:
        gate = normal_bf16((M, N), std, seed, device, gen)
        up = normal_bf16((M, N), std, seed, device, gen)
    dh = normal_bf16((M, N), std, seed, device, gen)
    if outlier_rate > 0:
        for t in (gate, up, dh):
            add_outliers_(t, outlier_rate, outlier_factor, gen)
    if zero_tile_rate > 0:
        zero_tiles_((gate, up, dh), 32, zero_tile_rate, gen)
    return SwigluInputs(gate, up, dh, w13)


def expert_weights(E: int, N: int, K: int, *, seed: int, std: float = 0.02, device="cpu") -> torch.Tensor:
    """Expert weight stack (E, N, K) of N(0, std^2) bf16 values."""
    return normal_bf16((E, N, K), std, seed, device)


# The workloads, by what they are.  Distribution readings: "N(0, s)" means
# standard deviation s; dh uses the same distribution as gate/up.
WORKLOADS = {
    "swiglu_128x128": dict(M=128, N=128, seed=0, std=1.0),
    "swiglu_4096x2048_outliers": dict(M=4096, N=2048, seed=1, std=1.0, outlier_rate=1e-3,
                                      outlier_factor=100.0, zero_tile_rate=0.01),
    "swiglu_16384x7168_w13": dict(M=16384, N=7168, seed=2, std=0.5, packed=True),
    "swiglu_131072x8192_w13": dict(M=131072, N=8192, seed=4, std=1.0, packed=True),
}

EXPERT_WORKLOADS = {E: dict(E=E, N=8192, K=5120, seed=3 + E, std=0.02) for E in (1, 4, 16, 64)}


def workload(name: str, device="cpu") -> SwigluInputs:
    return swiglu_inputs(device=device, **WORKLOADS[name])


def expert_workload(E: int, device="cpu") -> torch.Tensor:
    cfg = dict(EXPERT_WORKLOADS[E])
    return expert_weights(cfg.pop("E"), cfg.pop("N"), cfg.pop("K"), device=device, **cfg)
