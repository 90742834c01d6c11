"""Seeded synthetic inputs shared by the GPU path and the oracle.

This module only draws random numbers; it holds none of the method's
arithmetic and imports neither the HIP binding nor the oracle.  Every tensor
is drawn with torch generators from a fixed seed so both sides see identical
bytes:

* codes: uniform integers 0..15, one per byte, ``u8[N][K]``;
* packed weights for the large shapes: uniform bytes 0..255 drawn directly,
  which is exactly two independent uniform codes per byte;
* group scales: binary16 of ``|N(0,1)| * 0.02``, ``[N][K/32]``, handed out as
  their uint16 bit patterns;
* activations: binary16 of ``N(0,1)``; the per-token residual input of the
  decode step is fp32 ``N(0,1)``.

Seeds follow ``BASE_SEED + 1000*config + 10*layer + tensor_id`` so every
tensor of every workload has its own stream.
"""
from __future__ import annotations

import torch

BASE_SEED = 20261202
GROUP = 32

# Llama-shaped model dimensions used by the decode workloads.
MODEL_DIMS = {
    "8b": dict(d=4096, H=32, Hkv=8, hd=128, dff=14336, n_layers=32),
    "70b": dict(d=8192, H=64, Hkv=8, hd=128, dff=28672, n_layers=80),
}

# tensor ids inside one layer
TID = {"qkv": 0, "o": 2, "gate_up": 4, "down": 6}


def seed_of(config: int, layer: int = 0, tensor_id: int = 0) -> int:
    return BASE_SEED + 1000 * config + 10 * layer + tensor_id


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def codes(N: int, K: int, seed: int) -> torch.Tensor:
    """Uniform 4-bit codes, one per byte (CPU, u8[N][K])."""
    return torch.randint(0, 16, (N, K), dtype=torch.uint8, generator=_gen(seed))


def random_bytes(N: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniform bytes u8[N][K/2]: two independent uniform codes per byte."""
    return torch.randint(0, 256, (N, K // 2), dtype=torch.uint8,
                         generator=_gen(seed, device), device=device)


def scales(N: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    """binary16 bit patterns of |N(0,1)|*0.02, as int16 [N][K/32]."""
    r = torch.randn((N, K // GROUP), generator=_gen(seed, device), device=device)
    return (r.abs_().mul_(0.02)).to(torch.float16).view(torch.int16)


def act_f16(shape, seed: int, device="cpu") -> torch.Tensor:
    """binary16 bit patterns of N(0,1) activations (int16)."""
    if isinstance(shape, int):
        shape = (shape,)
    r = torch.randn(shape, generator=_gen(seed, device), device=device)
    return r.to(torch.float16).view(torch.int16)


def residual_f32(d: int, seed: int, device="cpu") -> torch.Tensor:
    """Per-token fp32 residual input, N(0,1)."""
    return torch.randn((d,), generator=_gen(seed, device), device=device)


def layer_shapes(dims: dict) -> dict:
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    return {"qkv": ((H + 2 * Hkv) * hd, d), "o": (d, H * hd),
            "gate_up": (2 * dff, d), "down": (d, dff)}


def layer_weights(dims: dict, config: int, layer: int, device="cpu") -> dict:
    """Random packed weights and scales of one decoder layer.

    Returns name -> (packed u8[N][K/2], scales int16[N][K/32]).
    """
    out = {}
    for name, (N, K) in layer_shapes(dims).items():
        t = TID[name]
        out[name] = (random_bytes(N, K, seed_of(config, layer, t), device),
                     scales(N, K, seed_of(config, layer, t + 1), device))
    return out


def to_numpy_u16(t: torch.Tensor):
    """binary16 bit patterns (int16 tensor, any device) -> numpy uint16."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
