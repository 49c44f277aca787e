"""Cache writer: bf16 latent + bf16 rope -> 656-byte fp8_ds_mla records.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from two sources:
* the writer rule the FlyDSL page states for vLLM's fp8_ds_mla cache writer
  (module docstring, section "Preconditions the host cannot check"): per 128
  latent values, scale = pow2ceil(max(amax, 1e-4) / 448), stored as an f32
  power of two; the latent values are stored as e4m3 codes of x / scale, the
  64 rope values as bf16, in the 656-byte record layout (module docstring);
* the OCP FP8 E4M3 ("FN") format: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, largest finite magnitude 448, conversion by rounding to the
  nearest value with ties to the even mantissa.

Everything is computed in fp64.  x / scale is exact there (x is a bf16 value
and the scale a power of two), so the only rounding is the e4m3 one.
"""

from __future__ import annotations

import numpy as np

from .codec import (
    LATENT_PER_SCALE,
    N_LATENT,
    N_ROPE,
    RECORD_BYTES,
    ROPE_BYTE0,
    SCALE_BYTE0,
    bf16_bits_to_f64,
)

AMAX_FLOOR = 1e-4
E4M3_MAX = 448.0


def pow2ceil(x) -> np.ndarray:
    """Smallest power of two >= x, for positive finite x (exact at powers of two)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~(x > 0)) or np.any(~np.isfinite(x)):
        raise ValueError("pow2ceil needs positive finite values")
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= m < 1
    return np.ldexp(1.0, np.where(m == 0.5, e - 1, e).astype(np.int64))


def e4m3_encode(y) -> np.ndarray:
    """OCP E4M3 codes (uint8) of finite values with |y| <= 448, rounded to the
    nearest e4m3 value with ties to the even mantissa.  The sign is kept
    (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode needs finite values with |y| <= 448")
    sign = np.signbit(y).astype(np.uint32)
    a = np.abs(y)
    # normal range, a >= 2^-6: a = (1 + f) * 2^(E - 7), f = mant / 8
    m, e = np.frexp(np.where(a > 0, a, 1.0))  # a = m 2^e, m in [0.5, 1): a = (2m) 2^(e-1)
    E = (e - 1 + 7).astype(np.int64)
    mant = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)  # np.rint: ties to even
    carry = mant == 8
    E = np.where(carry, E + 1, E)
    mant = np.where(carry, 0, mant)
    normal_code = (E << 3) | mant
    # subnormal range, a < 2^-6: a = mant * 2^-9 (mant = 8 is the smallest normal, code 8)
    sub_code = np.rint(a * 512.0).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, normal_code, sub_code)
    if np.any((code & 0x7F) == 0x7F) or np.any(code > 0x7F):
        raise AssertionError("rounded past 448")  # excluded by the range check
    return ((sign << 7) | code.astype(np.uint32)).astype(np.uint8)


def block_scales(latent: np.ndarray) -> np.ndarray:
    """[n, 512] float64 latent -> [n, 4] float64 scales by the writer rule."""
    n = latent.shape[0]
    amax = np.abs(latent.reshape(n, N_LATENT // LATENT_PER_SCALE, LATENT_PER_SCALE)).max(axis=2)
    return pow2ceil(np.maximum(amax, AMAX_FLOOR) / E4M3_MAX)


def encode_records(latent_bits, rope_bits) -> np.ndarray:
    """bf16 bit patterns: latent [n, 512], rope [n, 64] (uint16) -> uint8 records [n, 656]."""
    lb = np.asarray(latent_bits).astype(np.uint16)
    rb = np.asarray(rope_bits).astype(np.uint16)
    if lb.ndim != 2 or lb.shape[1] != N_LATENT or rb.shape != (lb.shape[0], N_ROPE):
        raise ValueError("latent must be [n, 512] and rope [n, 64] bf16 bits")
    n = lb.shape[0]
    x = bf16_bits_to_f64(lb)
    if not np.all(np.isfinite(x)):
        raise ValueError("latent values must be finite")
    scale = block_scales(x)                                  # [n, 4]
    y = x / np.repeat(scale, LATENT_PER_SCALE, axis=1)       # exact
    rec = np.zeros((n, RECORD_BYTES), np.uint8)
    rec[:, :N_LATENT] = e4m3_encode(y)
    rec[:, SCALE_BYTE0:ROPE_BYTE0] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, ROPE_BYTE0:] = rb.astype("<u2").view(np.uint8).reshape(n, 2 * N_ROPE)
    return rec


def write_cache(kv: np.ndarray, latent_bits, rope_bits, slots) -> np.ndarray:
    """A copy of kv [N, 656] with record slots[i] replaced by the encoding of
    token i; negative slots and slots >= N are skipped (no write)."""
    out = np.array(kv, dtype=np.uint8, copy=True)
    rec = encode_records(latent_bits, rope_bits)
    slots = np.asarray(slots, dtype=np.int64)
    for i, s in enumerate(slots):
        if 0 <= s < out.shape[0]:
            out[s] = rec[i]
    return out
