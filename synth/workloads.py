"""Seeded synthetic workloads shaped like the sparse-MLA decode problem.

Record layout written here (656 bytes per KV row), as the vLLM/FlyDSL page's
module docstring states it ("Record (656 B)"): bytes 0..511 are 512 e4m3
latent codes, bytes 512..527 four little-endian f32 power-of-two scales (one
per 128 latent values), bytes 528..655 sixty-four bf16 rope values.

The per-128 scale is the writer's rule quoted on the same page (section
"Preconditions the host cannot check"): scale = pow2ceil(max(amax, 1e-4)/448),
so every code satisfies |x / scale| <= 448 and no code saturates.  The e4m3
rounding itself is torch's float8_e4m3fn cast (round to nearest even); the
oracle never relies on how a code was rounded, only on the stored bytes.

Random streams (fixed order, so a seed fixes every byte):
  * ``gen_data`` (on the device the tensors are made on): q, then per chunk of
    records: latent, outlier mask and signs (only if outliers are requested),
    rope.
  * ``gen_idx`` (always CPU): row lengths (ragged configs), then per row the
    distinct indices.
"""

from __future__ import annotations

import math
import re
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np
import torch

RECORD_BYTES = 656
LATENT = 512
ROPE = 64
QK_DIM = LATENT + ROPE
BLOCK = 128  # latent values per scale
SCALE_OFF = 512
ROPE_OFF = 528
E4M3_MAX = 448.0
AMAX_FLOOR = 1e-4

# Records generated per chunk: bounds host/device temporaries to ~1 GiB.
_CHUNK = 1 << 18


@dataclass
class Workload:
    """One problem instance.  All tensors live on the same device."""

    name: str
    T: int
    H: int
    N: int
    q: torch.Tensor  # bf16 [T, H, 576]
    kv: torch.Tensor  # uint8 [N, 656]
    indptr: torch.Tensor  # int32 [T + 1]
    indices: torch.Tensor  # int32 [nnz]
    sm_scale: float  # exactly representable in f32
    has_invalid: int
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.indices.numel())

    def valid_entries(self) -> int:
        """Entries with index >= 0 inside their row's slice (the gathered rows)."""
        ip = self.indptr.cpu().numpy().astype(np.int64)
        ix = self.indices.cpu().numpy()
        n = 0
        for r in range(self.T):
            b, e = ip[r], ip[r + 1]
            if e > b:
                n += int((ix[b:e] >= 0).sum())
        return n

    def to(self, device) -> "Workload":
        return Workload(
            self.name, self.T, self.H, self.N, self.q.to(device), self.kv.to(device),
            self.indptr.to(device), self.indices.to(device), self.sm_scale,
            self.has_invalid, dict(self.meta),
        )


def f32(x: float) -> float:
    """Round a Python float to the nearest f32 value (what the C ABI receives)."""
    return float(np.float32(x))


def _pow2ceil(x: torch.Tensor) -> torch.Tensor:
    """Smallest power of two >= x, for positive f32 x (exact at powers of two)."""
    m, e = torch.frexp(x)  # x = m * 2**e, m in [0.5, 1)
    e = torch.where(m == 0.5, e - 1, e)
    return torch.ldexp(torch.ones_like(x), e)


def encode_records(latent: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
    """Pack f32 latent [n, 512] and f32 rope [n, 64] into uint8 records [n, 656]."""
    n = latent.shape[0]
    lat = latent.float().reshape(n, LATENT // BLOCK, BLOCK)
    amax = lat.abs().amax(dim=2)
    floor = torch.tensor(AMAX_FLOOR, dtype=torch.float32, device=lat.device)
    scale = _pow2ceil(torch.maximum(amax, floor) / E4M3_MAX)  # [n, 4] f32
    codes = (lat / scale[:, :, None]).reshape(n, LATENT).to(torch.float8_e4m3fn)
    rec = torch.empty(n, RECORD_BYTES, dtype=torch.uint8, device=lat.device)
    rec[:, :SCALE_OFF] = codes.view(torch.uint8)
    rec[:, SCALE_OFF:ROPE_OFF] = scale.contiguous().view(torch.uint8).reshape(n, 16)
    rec[:, ROPE_OFF:] = rope.to(torch.bfloat16).contiguous().view(torch.uint8).reshape(n, 2 * ROPE)
    return rec


def _make_records(N: int, gen: torch.Generator, device, latent_std: float,
                  outlier_p: float, outlier_mag: float) -> torch.Tensor:
    kv = torch.empty(N, RECORD_BYTES, dtype=torch.uint8, device=device)
    for s in range(0, N, _CHUNK):
        n = min(_CHUNK, N - s)
        lat = torch.randn(n, LATENT, generator=gen, device=device) * latent_std
        if outlier_p > 0.0:
            hit = torch.rand(n, LATENT, generator=gen, device=device) < outlier_p
            sign = torch.where(torch.rand(n, LATENT, generator=gen, device=device) < 0.5,
                               -1.0, 1.0)
            lat = torch.where(hit, sign * outlier_mag, lat)
        rope = torch.randn(n, ROPE, generator=gen, device=device)
        kv[s:s + n] = encode_records(lat, rope)
        del lat, rope
    return kv


def distinct_uniform(gen: torch.Generator, M: int, k: int) -> np.ndarray:
    """k distinct integers uniform over [0, M), in draw order (CPU generator)."""
    if k > M:
        raise ValueError(f"cannot draw {k} distinct values from [0, {M})")
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    if M <= 8 * k:
        return torch.randperm(M, generator=gen)[:k].numpy().astype(np.int64)
    have = np.zeros(0, dtype=np.int64)
    while have.size < k:
        need = k - have.size
        draw = torch.randint(0, M, (need + need // 8 + 8,), generator=gen).numpy()
        draw = draw[~np.isin(draw, have)]
        _, first = np.unique(draw, return_index=True)
        draw = draw[np.sort(first)]
        have = np.concatenate([have, draw[:need]])
    return have


RowFn = Callable[[torch.Generator, int, dict], np.ndarray]


def build_workload(name: str, T: int, H: int, N: int, rows: RowFn, *, seed: int,
                   sm_scale: Optional[float] = None, has_invalid: int = 0,
                   latent_std: float = 1.0, outlier_p: float = 0.0,
                   outlier_mag: float = 1000.0, device="cpu",
                   lengths: Optional[Callable[[torch.Generator], np.ndarray]] = None,
                   q_std: float = 1.0) -> Workload:
    """Generic builder.  ``rows(gen_idx, r, meta)`` returns row r's index slice
    (int64, -1 allowed); ``lengths(gen_idx)`` (optional) is drawn before any row
    and stored as ``meta["lengths"]``."""
    device = torch.device(device)
    gen_data = torch.Generator(device=device)
    gen_data.manual_seed(seed)
    gen_idx = torch.Generator()
    gen_idx.manual_seed(seed + 0x5EED)
    q = (torch.randn(T, H, QK_DIM, generator=gen_data, device=device) * q_std).to(torch.bfloat16)
    kv = _make_records(N, gen_data, device, latent_std, outlier_p, outlier_mag)
    meta = {}
    if lengths is not None:
        meta["lengths"] = lengths(gen_idx)
    slices: List[np.ndarray] = []
    for r in range(T):
        slices.append(np.asarray(rows(gen_idx, r, meta), dtype=np.int64))
    indptr = np.zeros(T + 1, dtype=np.int64)
    indptr[1:] = np.cumsum([s.size for s in slices])
    idx = np.concatenate(slices) if slices else np.zeros(0, dtype=np.int64)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(QK_DIM)
    return Workload(
        name=name, T=T, H=H, N=N, q=q, kv=kv,
        indptr=torch.from_numpy(indptr.astype(np.int32)).to(device),
        indices=torch.from_numpy(idx.astype(np.int32)).to(device),
        sm_scale=f32(sm_scale), has_invalid=int(has_invalid), meta=meta,
    )


# ---------------------------------------------------------------------------
# The five workloads, numbered as in the benchmark table (1-based).
# ---------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="tiny_T1_H16_N1024_top128", T=1, H=16, N=1024, topk=128),
    2: dict(name="decode_T64_H16_N65536_top2048", T=64, H=16, N=65536, topk=2048),
    3: dict(name="ragged_T256_H16_N262144_top2048_invalid", T=256, H=16, N=262144, topk=2048),
    4: dict(name="largecache_T128_H16_N8388608_top2048", T=128, H=16, N=8388608, topk=2048),
    5: dict(name="prefill_T4096_H64_N32768_top2048_causal", T=4096, H=64, N=32768, topk=2048),
    # An additional workload (not one of the five): the causal prefill of one
    # 2,048-token prompt, where row r attends to tokens 0 .. r (r + 1 keys, padded
    # to 2,048 with -1): a wide-head batch of genuinely ragged rows.
    6: dict(name="prefill_T2048_H64_N2048_top2048_causal_ragged", T=2048, H=64, N=2048, topk=2048),
}


def make_config(cfg: int) -> dict:
    return dict(CONFIGS[cfg])


def heads_name(name: str, H: int) -> str:
    """A workload's name with its head count replaced by H."""
    return re.sub(r"_H\d+_", f"_H{H}_", name, count=1)


def make_workload(cfg: int, device="cpu", seed: Optional[int] = None,
                  T: Optional[int] = None, H: Optional[int] = None) -> Workload:
    """Build configuration ``cfg`` (1..5, or 6: the additional ragged causal
    prefill).  ``seed`` defaults to the config
    number.  ``T`` may shrink the number of query rows (rows keep the same
    recipe; for the causal config the row positions keep their full-size
    meaning, i.e. row r is still row r of a 4096-row batch).  ``H`` replaces
    the configuration's head count (same records and slices; q has H heads)."""
    c = make_config(cfg)
    seed = cfg if seed is None else seed
    Tf, Hc, N, k = c["T"], c["H"], c["N"], c["topk"]
    H = Hc if H is None else H
    T = Tf if T is None else T
    base = c["name"] if H == Hc else heads_name(c["name"], H)
    name = base if T == Tf else f"{base}[T={T}]"
    if cfg == 1:
        return build_workload(name, T, H, N, lambda g, r, m: distinct_uniform(g, N, k), seed=seed,
                              device=device)
    if cfg == 2:
        return build_workload(name, T, H, N,
                              lambda g, r, m: np.sort(distinct_uniform(g, N, k)), seed=seed,
                              device=device)
    if cfg == 3:
        def lengths(g):
            return torch.randint(1, k + 1, (T,), generator=g).numpy().astype(np.int64)

        def rows(g, r, meta):
            L = int(meta["lengths"][r])
            return np.concatenate([distinct_uniform(g, N, L), -np.ones(k - L, np.int64)])
        return build_workload(name, T, H, N, rows, seed=seed, has_invalid=1,
                              latent_std=2.0, outlier_p=0.01, outlier_mag=1000.0,
                              lengths=lengths, device=device)
    if cfg == 4:
        return build_workload(name, T, H, N, lambda g, r, m: distinct_uniform(g, N, k),
                              seed=seed, device=device)
    if cfg == 6:
        def rows(g, r, m):
            take = min(r + 1, k)
            return np.concatenate([np.arange(take, dtype=np.int64), -np.ones(k - take, np.int64)])
        return build_workload(name, T, H, N, rows, seed=seed, has_invalid=1, device=device)
    if cfg == 5:
        def rows(g, r, m):
            avail = min(r + N - Tf + 1, N)
            take = min(k, avail)
            return np.concatenate([distinct_uniform(g, avail, take),
                                   -np.ones(k - take, np.int64)])
        return build_workload(name, T, H, N, rows, seed=seed, has_invalid=1, device=device)
    raise ValueError(f"unknown config {cfg}")
