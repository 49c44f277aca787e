"""Record and element decoding, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* e4m3 follows the OCP FP8 E4M3 ("FN") encoding: 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits, no infinities, 0x7F / 0xFF are NaN, the
  largest finite magnitude is 448.  The FlyDSL page's writer rule divides by
  448, which fixes this variant (the FNUZ variant tops out at 240).
* bf16 is the upper half of an IEEE binary32 word.
* A record (FlyDSL page, module docstring, "Record (656 B)") is 512 e4m3
  latent codes, then four f32 power-of-two scales (scale b applies to latent
  values 128b .. 128b+127), then 64 bf16 rope values.  K is the whole
  576-value decoded record, V its first 512 values.
"""

from __future__ import annotations

import math

import numpy as np

RECORD_BYTES = 656
N_LATENT = 512
N_ROPE = 64
SCALE_BYTE0 = 512
ROPE_BYTE0 = 528
LATENT_PER_SCALE = 128


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (0..255) as a Python float (NaN for 0x7F/0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:  # subnormal: man/8 * 2^(1-7)
        return sign * math.ldexp(man, -9)
    return sign * math.ldexp(8 + man, exp - 10)  # (1 + man/8) * 2^(exp-7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_TABLE.setflags(write=False)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (any integer array) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint32) & 0xFFFF
    return (b << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _le_f32(b4: np.ndarray) -> np.ndarray:
    """[..., 4] little-endian bytes -> float64."""
    b = b4.astype(np.uint32)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    return word.astype(np.uint32).view(np.float32).astype(np.float64)


def decode_records(rec: np.ndarray) -> np.ndarray:
    """uint8 records [n, 656] -> float64 K [n, 576].

    latent_j = e4m3(rec[j]) * scale[j // 128] for j < 512, with scale[b] the
    f32 stored at bytes 512+4b .. 515+4b; K[512 + i] = bf16(rec[528+2i .. 529+2i]).
    """
    rec = np.asarray(rec, dtype=np.uint8)
    if rec.ndim != 2 or rec.shape[1] != RECORD_BYTES:
        raise ValueError(f"records must be [n, {RECORD_BYTES}] uint8, got {rec.shape}")
    n = rec.shape[0]
    codes = rec[:, :N_LATENT]
    scales = _le_f32(rec[:, SCALE_BYTE0:ROPE_BYTE0].reshape(n, 4, 4))  # [n, 4]
    lat = E4M3_TABLE[codes] * np.repeat(scales, LATENT_PER_SCALE, axis=1)
    lo = rec[:, ROPE_BYTE0::2].astype(np.uint32)
    hi = rec[:, ROPE_BYTE0 + 1::2].astype(np.uint32)
    rope = bf16_bits_to_f64(lo | (hi << 8))
    return np.concatenate([lat, rope], axis=1)
