"""The DeepSeek V4.1 key record and the fused output epilogue, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the K2-back page ("vllm.models.deepseek_v41.amd.mono.attention.back"):
  * ``key_rec``: a key's data (its 448 e4m3 nope bytes, then its 64 bf16
    rope values: 576 bytes) is at page + offset * 576, and its scale bytes at
    page + page_records * 576 + offset * 8, i.e. a page keeps its keys' data
    first and their 8-byte scale words after it;
  * ``stage_split``: nope dims 64c .. 64c+63 use scale byte c (seven of the
    eight bytes), applied as the power of two 2^(byte - 127) (E8M0); K is
    [nope * scale, rope] (512 dims) and V is the same 512 values (the P.V
    covers the rope dims 448.. too); the softmax runs in log2 units with the
    scale folded into the scores, which is the same softmax;
  * ``stage_combine``: the chunks merged with the sink folded in, the result
    rounded to bf16, the inverse GPT-J rotation of dims 448.. (pairs of
    adjacent dims (e, o) = (2i, 2i+1) of the rope part: e' = e cos + o sin,
    o' = o cos - e sin, with cos_i and sin_i at the token's position), then
    "vLLM's MXFP8" of every 32 values.
Key entries, pools, the sink and empty rows are as in ``oracle.paged``.

Readings taken where the pages leave a point open:
  * MXFP8 is not defined on the pages.  This is the OCP Microscaling (MX) v1.0
    rule for E4M3 elements: the block's shared scale is 2^E with
    E = floor(log2(amax)) - 8 (8 = the exponent of E4M3's largest normal,
    448 = 1.75 * 2^8), stored as the E8M0 byte E + 127; every element is
    y / 2^E rounded to the nearest E4M3 value (ties to even) after clamping to
    +-448 (values up to 2^9 can exceed 448: the page clamps too).  A block of
    zeros, or one whose E would fall below -127, gets byte 0 (2^-127).
  * cos/sin come as a table of f32 [position, 64]: 32 cos then 32 sin, one
    pair index i per rope pair; the position of each query row is an input.
  * the bf16 rounding precedes the rotation (the page rounds, then rotates);
    the rotation and the quantisation are exact here (fp64).
"""

from __future__ import annotations

import numpy as np

from .codec import E4M3_TABLE, bf16_bits_to_f64
from .writer import e4m3_encode

NOPE = 448
ROPE = 64
DIM = NOPE + ROPE            # 512: K and V
DATA_BYTES = NOPE + 2 * ROPE  # 576
SCALE_BYTES = 8               # per key, 7 used
SCALE_BLOCK = 64              # nope dims per scale byte
MX_BLOCK = 32
E4M3_EMAX = 8                 # 448 = 1.75 * 2^8
SLOT_MASK = 0x7FFFFFFF


def e8m0_value(b) -> np.ndarray:
    """Value 2^(b - 127) of E8M0 bytes 0..254 (255 is NaN in the format)."""
    b = np.asarray(b, dtype=np.int64)
    if np.any((b < 0) | (b > 255)):
        raise ValueError("E8M0 bytes are 0..255")
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def decode_v41(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """data uint8 [n, 576] and scale bytes uint8 [n, 8] -> K (= V) float64 [n, 512]."""
    data = np.asarray(data, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if data.ndim != 2 or data.shape[1] != DATA_BYTES or scales.shape != (data.shape[0], SCALE_BYTES):
        raise ValueError("data must be [n, 576] and scales [n, 8]")
    n = data.shape[0]
    sc = e8m0_value(scales[:, : NOPE // SCALE_BLOCK])                 # [n, 7]
    nope = E4M3_TABLE[data[:, :NOPE]] * np.repeat(sc, SCALE_BLOCK, axis=1)
    rope = bf16_bits_to_f64(data[:, NOPE:].copy().view("<u2").reshape(n, ROPE))
    return np.concatenate([nope, rope], axis=1)


def resolve_v41(entry: int, pools):
    """(pool, data byte offset, scale byte offset) of a key-table entry, or
    None for -1.  pools: [(bytes, page_stride, page_records)] x 2."""
    entry = int(entry)
    if entry == -1:
        return None
    p = 0 if entry >= 0 else 1
    slot = entry & SLOT_MASK
    buf, stride, per_page = pools[p]
    page, off = divmod(slot, per_page)
    data = page * stride + off * DATA_BYTES
    scale = page * stride + per_page * DATA_BYTES + off * SCALE_BYTES
    if max(data + DATA_BYTES, scale + SCALE_BYTES) > len(buf):
        raise IndexError("slot past the pool (a precondition of the method)")
    return p, data, scale


def gather_v41(pools, entries):
    """(data [n, 576], scales [n, 8]) of the entries that are keys, in order."""
    ds, ss = [], []
    for e in entries:
        r = resolve_v41(e, pools)
        if r is not None:
            p, d, s = r
            buf = pools[p][0]
            ds.append(np.asarray(buf[d:d + DATA_BYTES], dtype=np.uint8))
            ss.append(np.asarray(buf[s:s + SCALE_BYTES], dtype=np.uint8))
    if not ds:
        return np.zeros((0, DATA_BYTES), np.uint8), np.zeros((0, SCALE_BYTES), np.uint8)
    return np.stack(ds), np.stack(ss)


def attention_v41(Q: np.ndarray, K: np.ndarray, sigma: float, sink):
    """Q [H, 512], K [n, 512] (V = K): softmax(sigma Q K^T) V with the sink as
    one more key of logit sink[h] and value 0.  Returns (out [H, 512], lse [H])."""
    H = Q.shape[0]
    sk = np.full(H, -np.inf) if sink is None else np.asarray(sink, np.float64).reshape(H)
    if K.shape[0] == 0:
        return np.zeros((H, DIM)), sk.copy()
    s = sigma * (Q @ K.T)
    m = np.maximum(s.max(axis=1), sk)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1) + np.exp(sk - m)
    return (p @ K) / l[:, None], m + np.log(l)


def sparse_mla_fwd_v41(q_bits, pools, indptr, indices, sm_scale, sink=None, rows=None):
    """Attention of bf16 q [T, H, 512] over V4.1 keys in two paged pools.
    Returns (out float64 [T, H, 512], lse float64 [T, H]); rows not in `rows` are NaN."""
    q_bits = np.asarray(q_bits)
    T, H, D = q_bits.shape
    if D != DIM:
        raise ValueError("q must be [T, H, 512]")
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    sigma = float(np.float32(sm_scale))
    out = np.full((T, H, DIM), np.nan)
    lse = np.full((T, H), np.nan)
    for r in (range(T) if rows is None else rows):
        b, e = int(indptr[r]), int(indptr[r + 1])
        sl = indices[b:e] if e > b else indices[0:0]
        data, scales = gather_v41(pools, sl)
        out[r], lse[r] = attention_v41(bf16_bits_to_f64(q_bits[r]), decode_v41(data, scales), sigma, sink)
    return out, lse


def bf16_round(x) -> np.ndarray:
    """float64 -> the nearest bf16 value (ties to even), as float64.  Finite inputs."""
    # round the f64 value to bf16 directly: a bf16 has 8 significant bits
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) >= 2.0 ** 128):
        raise ValueError("bf16_round needs finite values inside bf16's range")
    m, e = np.frexp(x)                                  # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)        # 8 significant bits, ties to even
    # bf16 subnormals (|x| < 2^-126) keep a fixed step of 2^-133
    sub = np.abs(x) < 2.0 ** -126
    r = np.where(sub, np.rint(np.ldexp(x, 133)) * 2.0 ** -133, r)
    return np.where(x == 0, x, r)


def inverse_rope_gptj(o: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """o [..., 512]; cos, sin [..., 32] (broadcast over heads).  Dims 448 + 2i,
    448 + 2i + 1 (i < 32) hold (e, o): e' = e cos_i + o sin_i,
    o' = o cos_i - e sin_i.  The nope dims pass through."""
    o = np.asarray(o, dtype=np.float64)
    y = o.copy()
    e_, od = o[..., NOPE::2], o[..., NOPE + 1::2]
    c = np.asarray(cos, np.float64)
    s = np.asarray(sin, np.float64)
    y[..., NOPE::2] = e_ * c + od * s
    y[..., NOPE + 1::2] = od * c - e_ * s
    return y


def mx_exponent(amax) -> np.ndarray:
    """Shared exponent E of MXFP8 (E4M3) blocks with largest magnitude amax:
    floor(log2(amax)) - 8, at least -127 (also for amax = 0)."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("amax must be finite and >= 0")
    _, e = np.frexp(np.where(a > 0, a, 1.0))           # a = m 2^e, m in [0.5, 1): floor(log2 a) = e - 1
    E = (e - 1) - E4M3_EMAX
    return np.where(a > 0, np.maximum(E, -127), -127).astype(np.int64)


def mxfp8_quantize(y: np.ndarray):
    """y [..., 32k] -> (E4M3 codes uint8 [..., 32k], E8M0 bytes uint8 [..., k])."""
    y = np.asarray(y, dtype=np.float64)
    if y.shape[-1] % MX_BLOCK:
        raise ValueError("the last dimension must be a multiple of 32")
    blocks = y.reshape(y.shape[:-1] + (y.shape[-1] // MX_BLOCK, MX_BLOCK))
    E = mx_exponent(np.abs(blocks).max(axis=-1))                 # [..., k]
    scaled = blocks / np.ldexp(1.0, E)[..., None]                # exact (power of two)
    codes = e4m3_encode(np.clip(scaled, -448.0, 448.0))
    return codes.reshape(y.shape), (E + 127).astype(np.uint8)


def mxfp8_dequantize(codes, e8m0) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    vals = E4M3_TABLE[codes].reshape(codes.shape[:-1] + (codes.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (vals * e8m0_value(e8m0)[..., None]).reshape(codes.shape)


def v41_epilogue(out: np.ndarray, cos_sin: np.ndarray, pos: np.ndarray):
    """out [T, H, 512] (the attention result), cos_sin f32 [P, 64], pos int [T]
    -> (y float64 [T, H, 512] before quantisation, codes uint8, e8m0 uint8).
    y = inverse GPT-J rotation of bf16(out) at each row's position."""
    cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(pos, dtype=np.int64)]   # [T, 64]
    y = inverse_rope_gptj(bf16_round(out), cs[:, None, :ROPE // 2], cs[:, None, ROPE // 2:])
    codes, e8 = mxfp8_quantize(y)
    return y, codes, e8
