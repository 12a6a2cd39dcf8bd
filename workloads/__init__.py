"""Seeded synthetic inputs for the quantizer workloads.

This module only draws random numbers and rounds them to bf16 input bits (with
torch's CPU fp32->bf16 conversion).  It holds none of the quantizers'
arithmetic; both the CPU oracle and the HIP library consume exactly the bits it
returns, so a parity check compares the two on identical inputs.

Workloads (shapes from the weights and activations the pages quantize: a
DeepSeek-style hidden size of 7168 and MoE expert width 2048):

  mx_small      bf16 [256, 512], N(0,1), seed 0, with injected edge groups
  weight_4097   bf16 [4097, 7168], N(0, 0.02), 0.1% of entries x100, seed 2
  act_16384     bf16 [16384, 7168], 0.5 * Student-t(3), seed 3
  moe_experts   128 experts x {gate [2048,7168], up [2048,7168], down [7168,2048]},
                N(0, 0.02 * u_e), u_e ~ U(0.5, 2) per expert, seed 4
  square_8192   bf16 [8192, 8192], N(0,1), 0.01% of entries x1000, seed 5

numpy's PCG64 ``default_rng(seed)`` draws everything except the expert
tensors; those are too large to draw on the host in a few seconds, so each is
drawn on the target device by a torch generator seeded with
``seed * 1000 + tensor_index`` (the bits then depend on the device type; the
oracle always receives a copy of the bits the device holds).
"""
from __future__ import annotations

import numpy as np
import torch

SHAPES = {
    "mx_small": (256, 512),
    "weight_4097": (4097, 7168),
    "act_16384": (16384, 7168),
    "square_8192": (8192, 8192),
}
SEEDS = {"mx_small": 0, "weight_4097": 2, "act_16384": 3, "moe_experts": 4, "square_8192": 5}

MOE_EXPERTS = 128
MOE_HIDDEN = 7168
MOE_INTER = 2048


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (torch CPU, round-to-nearest-even) and return the bits as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_from_float(v: float) -> int:
    return int(bf16_bits(np.array([[v]], np.float32))[0, 0])


def mx_small(seed: int = SEEDS["mx_small"]) -> np.ndarray:
    """[256, 512] N(0,1) with edge groups (group k of row k = columns 32k..32k+31):
    row 0 group 0 all zero; row 1 group 1 all 1e-30 with alternating signs;
    row 2 group 2 one +1e4; row 3 group 3 one -1e4; row 4 group 4 holds 448 and 449."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(SHAPES["mx_small"], dtype=np.float32)
    x[0, 0:32] = 0.0
    x[1, 32:64] = 1e-30 * np.where(np.arange(32) % 2 == 0, 1.0, -1.0)
    x[2, 64 + 5] = 1e4
    x[3, 96 + 17] = -1e4
    x[4, 128 + 3] = 448.0
    x[4, 128 + 4] = 449.0
    return bf16_bits(x)


def weight_4097(seed: int = SEEDS["weight_4097"]) -> np.ndarray:
    rng = np.random.default_rng(seed)
    shape = SHAPES["weight_4097"]
    x = rng.normal(0.0, 0.02, size=shape).astype(np.float32)
    mask = rng.random(size=shape) < 1e-3
    x[mask] *= 100.0
    return bf16_bits(x)


def act_16384(seed: int = SEEDS["act_16384"], rows: int | None = None) -> np.ndarray:
    """0.5 * Student-t(df=3); ``rows`` draws a leading slice of the same recipe (smaller tests)."""
    rng = np.random.default_rng(seed)
    r, c = SHAPES["act_16384"]
    r = r if rows is None else rows
    x = (0.5 * rng.standard_t(3, size=(r, c))).astype(np.float32)
    return bf16_bits(x)


def square_8192(seed: int = SEEDS["square_8192"], n: int | None = None) -> np.ndarray:
    rng = np.random.default_rng(seed)
    shape = SHAPES["square_8192"] if n is None else (n, n)
    x = rng.standard_normal(shape, dtype=np.float32)
    mask = rng.random(size=shape) < 1e-4
    x[mask] *= 1000.0
    return bf16_bits(x)


def moe_shapes(experts: int = MOE_EXPERTS, hidden: int = MOE_HIDDEN, inter: int = MOE_INTER):
    """Expert-major list of (name, rows, cols): gate [inter, hidden], up [inter, hidden], down [hidden, inter]."""
    out = []
    for e in range(experts):
        out.append((f"experts.{e}.gate_proj.weight", inter, hidden))
        out.append((f"experts.{e}.up_proj.weight", inter, hidden))
        out.append((f"experts.{e}.down_proj.weight", hidden, inter))
    return out


def moe_multipliers(experts: int = MOE_EXPERTS, seed: int = SEEDS["moe_experts"]) -> np.ndarray:
    """Per-expert std multiplier u_e ~ U(0.5, 2), drawn first."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 2.0, size=experts)


def moe_tensor(index: int, rows: int, cols: int, multiplier: float, device,
               seed: int = SEEDS["moe_experts"]) -> torch.Tensor:
    """One expert tensor, N(0, 0.02 * u_e), drawn on ``device`` and rounded to bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + index)
    t = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    t.mul_(0.02 * float(multiplier))
    return t.to(torch.bfloat16)


def random_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Generic N(0, std) bf16 bits for ragged/edge-case parity shapes."""
    rng = np.random.default_rng(seed)
    return bf16_bits((std * rng.standard_normal(shape)).astype(np.float32))
