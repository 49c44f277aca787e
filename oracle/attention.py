"""Sparse MLA forward, written as its plain definition in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the method computes (FlyDSL page, module docstring and kernel epilogue):
for every query row r and head h, softmax attention of the bf16 query row
q[r, h, :576] over the KV records listed in the row's CSR slice
indices[indptr[r] : indptr[r+1]], with K the 576-value decoded record, V its
512 latent values and the logits scaled by sm_scale.  The kernel also returns
the natural-log log-sum-exp of the scaled logits.

Readings taken where the pages leave a point open:
  * an entry < 0 is "no key" whether or not the caller sets has_invalid
    (has_invalid only lets the kernel skip trailing tiles), so the oracle has
    no has_invalid argument;
  * a row whose slice is empty, negative-length or all negative gets out = 0
    and lse = -inf (the page's epilogue: zero output when the softmax sum is
    zero, -inf LSE when no key is unmasked);
  * duplicate indices count once per CSR entry;
  * an index >= the number of records breaks a stated precondition: raise.
"""

from __future__ import annotations

import numpy as np

from .codec import N_LATENT, bf16_bits_to_f64, decode_records


def row_attention(Q: np.ndarray, K: np.ndarray, sigma: float, with_abs: bool = False):
    """Softmax attention of Q [H, 576] over keys K [n, 576], values K[:, :512].

    Returns (out [H, 512], lse [H]) in float64; n == 0 gives (0, -inf).
    s = sigma * Q K^T;  m = max_j s;  p = exp(s - m);  l = sum_j p;
    out = p V / l;  lse = m + ln l.
    with_abs: also return A = p |V| / l, the softmax-weighted mean of |V| per
    output element (0 for n == 0).  It scales the rounding error of any
    evaluation that rounds the weights p to a short format before the p V
    product (the tests' error bound uses it).
    """
    H = Q.shape[0]
    if K.shape[0] == 0:
        empty = (np.zeros((H, N_LATENT)), np.full(H, -np.inf))
        return empty + (np.zeros((H, N_LATENT)),) if with_abs else empty
    s = sigma * (Q @ K.T)  # [H, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    out = (p @ K[:, :N_LATENT]) / l[:, None]
    lse = m[:, 0] + np.log(l)
    if with_abs:
        return out, lse, (p @ np.abs(K[:, :N_LATENT])) / l[:, None]
    return out, lse


def _row_keys(kv: np.ndarray, slice_: np.ndarray) -> np.ndarray:
    kept = slice_[slice_ >= 0]
    if kept.size and int(kept.max()) >= kv.shape[0]:
        raise IndexError("index >= number of KV records (a precondition of the method)")
    return decode_records(kv[kept])


def sparse_mla_fwd(q_bits: np.ndarray, kv: np.ndarray, indptr: np.ndarray,
                   indices: np.ndarray, sm_scale: float, rows=None, with_abs: bool = False):
    """Oracle forward.

    q_bits  : bf16 bit patterns [T, H, 576] (uint16 or int16)
    kv      : uint8 [N, 656]
    indptr  : int [T + 1]; indices: int [nnz]
    sm_scale: the f32 value the C ABI receives (used as float64)
    rows    : optional iterable of row numbers to compute (others stay NaN)

    Returns (out float64 [T, H, 512], lse float64 [T, H]), and with with_abs
    also A float64 [T, H, 512] (see row_attention).
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
    absw = np.full((T, H, N_LATENT), np.nan) if with_abs else None
    for r in (range(T) if rows is None else rows):
        b, e = int(indptr[r]), int(indptr[r + 1])
        sl = indices[b:e] if e > b else indices[0:0]
        K = _row_keys(kv, sl)
        res = row_attention(bf16_bits_to_f64(q_bits[r]), K, sigma, with_abs=with_abs)
        out[r], lse[r] = res[0], res[1]
        if with_abs:
            absw[r] = res[2]
    return (out, lse, absw) if with_abs else (out, lse)


def lse_merge(parts):
    """Merge chunk results of one (row, head) set into the whole-row result.

    parts: list of (out_c [..., 512], lse_c [...]) from disjoint chunks of the
    same key set.  This is the combine of the K2-back page (``stage_combine``:
    the chunks' maxima and sums re-weighted to a common maximum), written in
    the normalized form: with M = max_c lse_c and w_c = exp(lse_c - M),
    out = sum_c w_c out_c / sum_c w_c and lse = M + ln sum_c w_c.  Chunks with
    lse_c = -inf (no key) carry no weight; if every chunk is empty the result
    is (0, -inf).
    """
    outs = np.stack([np.asarray(o, dtype=np.float64) for o, _ in parts])
    lses = np.stack([np.asarray(s, dtype=np.float64) for _, s in parts])
    M = lses.max(axis=0)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms), 0.0)
    wsum = w.sum(axis=0)
    safe = np.where(wsum > 0, wsum, 1.0)
    out = np.where(live[..., None],
                   (w[..., None] * np.nan_to_num(outs)).sum(axis=0) / safe[..., None], 0.0)
    lse = np.where(live, Ms + np.log(safe), -np.inf)
    return out, lse
