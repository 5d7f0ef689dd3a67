"""Seeded synthetic inputs for the skinny decode projection.

Shared by the CPU oracle tests, the GPU parity tests and the benchmark, and
by nothing else.  It holds none of the projection's arithmetic: it draws
random numbers, stores them as bf16, and builds routing tables.  The same
tensor is handed to both sides of a parity check; neither side regenerates.

Recipes (the pages name no model dimensions; these are the workload shapes
used throughout):
  * activations x ~ N(0, sigma_x^2), weights W ~ N(0, 0.02^2), residual
    r ~ N(0, 1): float32 normals from a seeded torch.Generator, scaled, then
    rounded to bf16 by torch's round-to-nearest-even conversion;
  * routing: for each token in order, the first ``topk`` entries of a seeded
    random permutation of the E expert ids (distinct, uniform);
  * integer-valued tensors: uniform integers in [lo, hi] stored as bf16 (all
    exactly representable), for the exact-sum checks;
  * MXFP4 weights: uniform random bytes (two 4-bit codes each) and uniform
    random 8-bit block scales in a band (by default 119..121, so weights of
    magnitude about 0.02 like the bf16 ones).
Seeds: workload c uses base 1000*c; tags add x:+0, W:+1 (expert e: +100+e),
r:+2, routing:+3 (routing table i of a ring: +3+10*i).
"""
from __future__ import annotations

import torch

WEIGHT_SIGMA = 0.02

TAG_X, TAG_W, TAG_R, TAG_ROUTING = 0, 1, 2, 3


def seed_for(workload: int, tag: int) -> int:
    return 1000 * workload + tag


def _generator(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, sigma: float, seed: int, device: str = "cpu") -> torch.Tensor:
    """bf16 tensor of N(0, sigma^2) draws (float32 draw, then RNE to bf16)."""
    g = _generator(seed, device)
    v = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return (v * sigma).to(torch.bfloat16)


def integer_bf16(shape, lo: int, hi: int, seed: int, device: str = "cpu") -> torch.Tensor:
    """bf16 tensor of uniform integers in [lo, hi] (exact in bf16 for |v| <= 256)."""
    assert -256 <= lo <= hi <= 256
    g = _generator(seed, device)
    v = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return v.to(torch.bfloat16)


def routing_table(T: int, E: int, topk: int, seed: int) -> torch.Tensor:
    """int32 [T, topk]: per token, ``topk`` distinct expert ids drawn uniformly."""
    assert topk <= E
    g = _generator(seed, "cpu")
    rows = [torch.randperm(E, generator=g)[:topk] for _ in range(T)]
    if not rows:
        return torch.empty((0, topk), dtype=torch.int32)
    return torch.stack(rows).to(torch.int32)


def random_bytes(shape, lo: int, hi: int, seed: int, device: str = "cpu") -> torch.Tensor:
    """uint8 tensor of uniform integers in [lo, hi] (packed 4-bit codes, or scale codes)."""
    assert 0 <= lo <= hi <= 255
    g = _generator(seed, device)
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def mxfp4_weights(N: int, K: int, seed: int, device: str = "cpu", scale_lo: int = 119,
                  scale_hi: int = 121):
    """(codes uint8 [N, K/2], scales uint8 [N, K/32]): random 4-bit weight codes and
    block scale codes for a [N, K] MXFP4 weight matrix (K a multiple of 32)."""
    assert K % 32 == 0
    return (random_bytes((N, K // 2), 0, 255, seed, device),
            random_bytes((N, K // 32), scale_lo, scale_hi, seed + 7919, device))


def fp8_weights(N: int, K: int, seed: int, device: str = "cpu", scale_lo: float = 2e-5,
                scale_hi: float = 1e-4):
    """(codes uint8 [N, K], scales float32 [ceil(N/128), ceil(K/128)]): random e4m3 weight
    codes (the two NaN codes 0x7F and 0xFF replaced by 0x00) and uniform block scales."""
    codes = random_bytes((N, K), 0, 255, seed, device)
    codes[(codes & 0x7F) == 0x7F] = 0
    g = _generator(seed + 104729, "cpu")
    shape = (-(-N // 128), -(-K // 128))
    scales = (torch.rand(shape, generator=g, dtype=torch.float32) * (scale_hi - scale_lo)
              + scale_lo).to(device)
    return codes, scales


def bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bf16 tensor, as a numpy array on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(a, device: str = "cpu") -> torch.Tensor:
    """bf16 tensor from raw uint16 bit patterns (numpy)."""
    import numpy as np
    a = np.ascontiguousarray(a).view(np.int16)
    return torch.from_numpy(a.copy()).view(torch.bfloat16).to(device)
