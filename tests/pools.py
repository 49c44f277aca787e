"""Paged two-pool layouts for the tests: scatter the records of a contiguous
cache over a window pool and a compressed pool and return the key-table entry
of every record (K2-back page, "key_rec": -1 no key, a value >= 0 a window
slot, a compressed slot with bit 31 set).  Pure input layout; the tests then
resolve entries with the oracle on one side and the library on the other."""

from __future__ import annotations

import numpy as np

RECORD_BYTES = 656


def compressed_entry(slot):
    """Key-table entry of compressed-pool slot `slot` (bit 31 set, as int32)."""
    return (np.asarray(slot, np.int64) | (1 << 31)).astype(np.uint32).view(np.int32).astype(np.int64)


def paged_layout(rng, kv, per_page=(16, 8), pad=(3 * 656 + 16, 0), pool_of=None):
    """Scatter the records of kv [N, 656] over two paged pools: each record
    goes to pool pool_of[i] (random when None) at a random slot; pages are
    page_stride = per_page * 656 + pad bytes apart and the gaps hold random
    bytes.  Returns (pools, entry_of): pools = [(bytes, page_stride,
    page_records)] x 2, entry_of[i] the key-table entry of record i."""
    kv = np.asarray(kv, np.uint8)
    N = kv.shape[0]
    pool_of = rng.integers(0, 2, N) if pool_of is None else np.asarray(pool_of)
    pools, entry_of = [], np.zeros(N, np.int64)
    for p in range(2):
        ids = np.flatnonzero(pool_of == p)
        slots = rng.permutation(max(len(ids), 1))[: len(ids)].astype(np.int64)
        blk = per_page[p]
        stride = blk * RECORD_BYTES + pad[p]
        npages = (int(slots.max()) // blk + 1) if len(ids) else 1
        buf = rng.integers(0, 256, npages * stride, dtype=np.uint8)
        if len(ids):
            off = (slots // blk) * stride + (slots % blk) * RECORD_BYTES
            buf[off[:, None] + np.arange(RECORD_BYTES)[None, :]] = kv[ids]
            entry_of[ids] = slots if p == 0 else compressed_entry(slots)
        pools.append((buf, stride, blk))
    return pools, entry_of


V41_DATA = 576
V41_SCALES = 8


def v41_layout(rng, data, scales, per_page=(16, 8), pad=(32, 0), pool_of=None):
    """Scatter V4.1 keys (data [N, 576], scale bytes [N, 8]) over two paged
    pools.  A page of r keys holds their data (r x 576 B) and then their scale
    words (r x 8 B), followed by `pad` random bytes (K2-back page, key_rec).
    Returns (pools, entry_of) like paged_layout."""
    data = np.asarray(data, np.uint8)
    scales = np.asarray(scales, np.uint8)
    N = data.shape[0]
    pool_of = rng.integers(0, 2, N) if pool_of is None else np.asarray(pool_of)
    pools, entry_of = [], np.zeros(N, np.int64)
    for p in range(2):
        ids = np.flatnonzero(pool_of == p)
        slots = rng.permutation(max(len(ids), 1))[: len(ids)].astype(np.int64)
        r = per_page[p]
        stride = r * (V41_DATA + V41_SCALES) + pad[p]
        npages = (int(slots.max()) // r + 1) if len(ids) else 1
        buf = rng.integers(0, 256, npages * stride, dtype=np.uint8)
        if len(ids):
            page, off = slots // r, slots % r
            d0 = page * stride + off * V41_DATA
            s0 = page * stride + r * V41_DATA + off * V41_SCALES
            buf[d0[:, None] + np.arange(V41_DATA)[None, :]] = data[ids]
            buf[s0[:, None] + np.arange(V41_SCALES)[None, :]] = scales[ids]
            entry_of[ids] = slots if p == 0 else compressed_entry(slots)
        pools.append((buf, stride, r))
    return pools, entry_of
