"""Paged two-pool key addressing and the attention sink, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the K2-back page ("vllm.models.deepseek_v41.amd.mono.attention.back"):
  * ``key_rec``: a key-table entry is -1 for "no key"; a value >= 0 is a slot
    of the window pool; a slot of the compressed pool has bit 31 set (slot |
    1 << 31, a negative int32 other than -1).  A pool is paged: page =
    slot // page_records, offset = slot % page_records, and the page starts
    at pool base + page * page_stride;
  * ``stage_combine``: the per-head sink is folded into the softmax: the
    maximum is max(m, sink) and the sum gains exp(sink - that maximum), i.e.
    the sink acts as one more key whose logit is sink_h and whose value is 0.

Readings taken where the pages leave a point open:
  * the record stays the 656-byte fp8_ds_mla record, whole, at page + offset
    * 656 (the page's layout that stores a page's scales after its data is
    part of its own V4.1 record format, not of this record);
  * sink is in natural-log logit units (the page scales it by log2 e before
    its exp2), one value per head; a row with no key gets out = 0 and
    lse = sink (-inf when there is no sink);
  * a slot whose record would lie past the pool's bytes breaks a precondition:
    raise.
"""

from __future__ import annotations

import numpy as np

from .codec import N_LATENT, RECORD_BYTES, bf16_bits_to_f64, decode_records

SLOT_MASK = 0x7FFFFFFF


def resolve(entry: int, pools):
    """(pool number, byte offset) of a key-table entry, or None for -1."""
    entry = int(entry)
    if entry == -1:
        return None
    p = 0 if entry >= 0 else 1
    slot = entry & SLOT_MASK
    _, stride, per_page = pools[p]
    off = (slot // per_page) * stride + (slot % per_page) * RECORD_BYTES
    if off + RECORD_BYTES > len(pools[p][0]):
        raise IndexError("slot past the pool (a precondition of the method)")
    return p, off


def gather_records(pools, entries) -> np.ndarray:
    """uint8 [n, 656] records of the entries that are keys (entry != -1), in order."""
    rows = []
    for e in entries:
        r = resolve(e, pools)
        if r is not None:
            p, off = r
            rows.append(np.asarray(pools[p][0][off:off + RECORD_BYTES], dtype=np.uint8))
    if not rows:
        return np.zeros((0, RECORD_BYTES), np.uint8)
    return np.stack(rows)


def row_attention_sink(Q: np.ndarray, K: np.ndarray, sigma: float, sink):
    """Softmax attention of Q [H, 576] over keys K [n, 576] (values K[:, :512])
    plus, per head h, one extra key of logit sink[h] and value 0.
    sink None: no extra key.  Returns (out [H, 512], lse [H]).

    s = sigma Q K^T;  m = max(max_j s, sink);  p = exp(s - m);
    l = sum_j p + exp(sink - m);  out = p V / l;  lse = m + ln l.
    """
    H = Q.shape[0]
    sk = np.full(H, -np.inf) if sink is None else np.asarray(sink, np.float64).reshape(H)
    if K.shape[0] == 0:
        return np.zeros((H, N_LATENT)), sk.copy()
    s = sigma * (Q @ K.T)
    m = np.maximum(s.max(axis=1), sk)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1) + np.exp(sk - m)
    out = (p @ K[:, :N_LATENT]) / l[:, None]
    return out, m + np.log(l)


def sparse_mla_fwd_paged(q_bits, pools, indptr, indices, sm_scale, sink=None, rows=None):
    """Oracle forward over two paged pools, with an optional sink.

    pools   : [(bytes uint8 1-D, page_stride bytes, page_records), x 2]
              (window pool, compressed pool)
    sink    : float [H] (natural-log logits) or None
    Other arguments as ``oracle.sparse_mla_fwd``.
    """
    q_bits = np.asarray(q_bits)
    T, H, D = q_bits.shape
    if D != 576:
        raise ValueError("q must be [T, H, 576]")
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    sigma = float(np.float32(sm_scale))
    out = np.full((T, H, N_LATENT), np.nan)
    lse = np.full((T, H), np.nan)
    for r in (range(T) if rows is None else rows):
        b, e = int(indptr[r]), int(indptr[r + 1])
        sl = indices[b:e] if e > b else indices[0:0]
        K = decode_records(gather_records(pools, sl))
        out[r], lse[r] = row_attention_sink(bf16_bits_to_f64(q_bits[r]), K, sigma, sink)
    return out, lse
