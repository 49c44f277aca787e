"""Seeded synthetic inputs for the DeepSeek V4.1 key record (K2-back page,
"vllm.models.deepseek_v41.amd.mono.attention.back": 448 e4m3 nope values and
64 bf16 rope values per key, one E8M0 scale byte per 64 nope values).

None of the method's arithmetic lives here: the keys are generated, quantised
by a stated recipe (the pages give no writer rule for this record) and handed
over as bytes; the oracle and the library decode them independently.

Recipe: nope values N(0, sigma^2) (optionally with outliers), rope values
N(0, 1) as bf16; per 64 nope values the scale is 2^e with
e = ceil(log2(max(amax, 2^-30) / 448)) (so amax / 2^e <= 448), stored as the
byte e + 127, and the codes are torch's float8_e4m3fn cast of x / 2^e
(round to nearest even).  The eighth scale byte is 0.
"""

from __future__ import annotations

import math

import numpy as np
import torch

NOPE = 448
ROPE = 64
DATA_BYTES = 576
SCALE_BYTES = 8


def make_v41_keys(N: int, seed: int, sigma: float = 1.0, outlier_p: float = 0.0,
                  outlier_mag: float = 1000.0):
    """(data uint8 [N, 576], scales uint8 [N, 8]) as numpy arrays."""
    g = torch.Generator()
    g.manual_seed(seed)
    x = torch.randn(N, NOPE, generator=g, dtype=torch.float64) * sigma
    if outlier_p > 0:
        hit = torch.rand(N, NOPE, generator=g, dtype=torch.float64) < outlier_p
        sign = torch.where(torch.rand(N, NOPE, generator=g) < 0.5, -1.0, 1.0).to(torch.float64)
        x = torch.where(hit, sign * outlier_mag, x)
    blocks = x.view(N, NOPE // 64, 64)
    amax = blocks.abs().amax(dim=2).clamp_min(2.0 ** -30)
    e = torch.ceil(torch.log2(amax / 448.0))
    # log2 rounding can leave amax / 2^e a hair above 448: step up then
    e = torch.where(amax / torch.exp2(e) > 448.0, e + 1, e)
    codes = (blocks / torch.exp2(e)[:, :, None]).to(torch.float32).to(torch.float8_e4m3fn)
    data = np.zeros((N, DATA_BYTES), np.uint8)
    data[:, :NOPE] = codes.view(torch.uint8).reshape(N, NOPE).numpy()
    rope = torch.randn(N, ROPE, generator=g).to(torch.bfloat16)
    data[:, NOPE:] = rope.view(torch.int16).numpy().view(np.uint8).reshape(N, 2 * ROPE)
    scales = np.zeros((N, SCALE_BYTES), np.uint8)
    scales[:, : NOPE // 64] = (e + 127).to(torch.int64).numpy().astype(np.uint8)
    return data, scales


def make_cos_sin(P: int, base: float = 10000.0) -> np.ndarray:
    """f32 [P, 64]: cos(p * theta_i) for i < 32, then sin(p * theta_i),
    theta_i = base^(-i / 32)."""
    i = np.arange(ROPE // 2, dtype=np.float64)
    theta = base ** (-i / (ROPE // 2))
    ang = np.arange(P, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_q(T: int, H: int, seed: int, std: float = 1.0) -> torch.Tensor:
    """bf16 [T, H, 512] query (rotated query of the page: an input here)."""
    g = torch.Generator()
    g.manual_seed(seed)
    return (torch.randn(T, H, NOPE + ROPE, generator=g) * std).to(torch.bfloat16)


def sm_scale_v41() -> float:
    return float(np.float32(1.0 / math.sqrt(NOPE + ROPE)))
