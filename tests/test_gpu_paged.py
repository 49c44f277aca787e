"""GPU parity of the paged two-pool forward with the attention sink
(sparse_mla_fwd_paged, through the C ABI) against the fp64 oracle
(oracle.sparse_mla_fwd_paged), plus bit-identity with the contiguous forward
when the same keys are reached through pages.

Readings checked here (K2-back page, "key_rec" and "stage_combine"): -1 is no
key, an entry >= 0 a window-pool slot, other negative entries compressed-pool
slots with bit 31 set; the sink is one more key per head with logit sink[h]
(natural log, not scaled) and value 0.  Every case prints its name before
touching the GPU.  Inputs are seeded and synthetic.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare, q_bits, sample_rows
from pools import compressed_entry, paged_layout

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_fp8_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield m
    m.set_option("split", 0)
    m.set_option("persist", 0)


def entries(w, entry_of):
    """The workload's contiguous indices mapped to key-table entries (-1 kept)."""
    ix = w.indices.cpu().numpy().astype(np.int64)
    return np.where(ix >= 0, entry_of[np.maximum(ix, 0)], -1)


def to_dev(pools):
    return [(None if b is None else torch.from_numpy(np.ascontiguousarray(b)).to(DEV), st, pr)
            for b, st, pr in pools]


def run_paged(smla, w, pools_d, ent, sink=None, has_invalid=None):
    hi = w.has_invalid if has_invalid is None else has_invalid
    sk = None if sink is None else torch.as_tensor(np.asarray(sink, np.float32)).to(DEV)
    o, l = smla.fwd_paged(w.q.to(DEV), pools_d, w.indptr.to(DEV),
                          torch.from_numpy(ent.astype(np.int32)).to(DEV), w.sm_scale,
                          sink=sk, has_invalid=bool(hi))
    torch.cuda.synchronize()
    return o, l


def run_oracle_paged(w, pools, ent, sink=None, rows=None):
    return oracle.sparse_mla_fwd_paged(q_bits(w), pools, w.indptr.cpu().numpy(), ent, w.sm_scale,
                                       sink=None if sink is None else np.asarray(sink, np.float64),
                                       rows=rows)


def ragged_workload(name, H, lens, N, seed, invalid_p=0.05, trailing=0):
    """Rows of the given lengths (distinct uniform keys), a fraction invalid_p
    of entries set to -1 and `trailing` -1 entries appended to every row."""
    def rows(g, r, m):
        L = lens[r]
        s = synth.distinct_uniform(g, N, L) if L else np.zeros(0, np.int64)
        if L:
            drop = torch.rand(L, generator=g).numpy() < invalid_p
            s = np.where(drop, -1, s)
        return np.concatenate([s, -np.ones(trailing, np.int64)])
    return synth.build_workload(name, len(lens), H, N, rows, seed=seed,
                                has_invalid=int(invalid_p > 0 or trailing > 0))


def sink_values(rng, H):
    """Per-head sinks: N(0, 3), with the edge cases -inf (no sink), a dominant
    +40 and a value near the typical logit."""
    s = rng.normal(0.0, 3.0, H)
    s[0] = -np.inf
    if H > 1:
        s[1] = 40.0
    if H > 2:
        s[2] = 0.5
    return s


@pytest.mark.parametrize("H", [16, 64, 5])
def test_paged_equals_contiguous_bitwise(smla, H):
    """Same keys reached through two paged pools: outputs and lse bit-identical
    to the contiguous forward (the kernels differ only in the record address)."""
    w = ragged_workload(f"paged_eq_H{H}", H, [1500, 129, 0, 2048, 7], 5000, seed=60 + H)
    rng = np.random.default_rng(61)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(64, 1), pad=(48, 0))
    ent = entries(w, entry_of)
    note(f"paged == contiguous H={H} T={w.T} nnz={w.nnz}")
    o_p, l_p = run_paged(smla, w, to_dev(pools), ent)
    wd = w.to(DEV)
    o_c, l_c = smla.fwd(wd.q, wd.kv, wd.indptr, wd.indices, w.sm_scale, has_invalid=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))
    assert torch.equal(l_p, l_c)


@pytest.mark.parametrize("H", [16, 64, 3, 128])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_paged_sink_matches_oracle(smla, H, split):
    """Both pools, -1 entries, an empty row, a one-key row and trailing padding;
    per-head sinks including -inf and a dominant one; automatic, no and forced
    splits (the combine folds the sink into split rows)."""
    lens = [0, 1, 129, 700, 2048, 333]
    w = ragged_workload(f"paged_sink_H{H}_S{split}", H, lens, 8000, seed=70 + H + split, trailing=40)
    rng = np.random.default_rng(71 + split)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(16, 8), pad=(3 * 656 + 16, 0))
    ent = entries(w, entry_of)
    sink = sink_values(rng, H)
    note(f"paged sink H={H} split={split} T={w.T}")
    smla.set_option("split", split)
    try:
        o, l = run_paged(smla, w, to_dev(pools), ent, sink=sink)
    finally:
        smla.set_option("split", 0)
    ro, rl = run_oracle_paged(w, pools, ent, sink=sink)
    compare(o, l, ro, rl, label=f"paged_sink_H{H}_S{split}")
    # the empty row: out 0 and lse = sink (split rows take it through log2
    # units and back: a few f32 ulps)
    assert torch.all(o[0] == 0)
    np.testing.assert_allclose(l[0].cpu().numpy(), sink.astype(np.float32), rtol=2e-6, atol=0)


@pytest.mark.parametrize("H,split", [(16, 0), (64, 0), (64, 3), (128, 2)])
def test_paged_uniform_rows(smla, H, split):
    """Rows of one length (so nnz is a multiple of T and every unit guesses
    its slice start and queues its first index tiles before indptr arrives),
    with -1 entries: through both pools, with sinks, against the oracle."""
    w = ragged_workload(f"paged_uni_H{H}_S{split}", H, [700] * 6, 8000, seed=90 + H + split)
    assert w.nnz % w.T == 0
    rng = np.random.default_rng(91 + split)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(16, 8), pad=(3 * 656 + 16, 0))
    ent = entries(w, entry_of)
    sink = sink_values(rng, H)
    note(f"paged uniform rows H={H} split={split} T={w.T}")
    smla.set_option("split", split)
    try:
        o, l = run_paged(smla, w, to_dev(pools), ent, sink=sink)
    finally:
        smla.set_option("split", 0)
    ro, rl = run_oracle_paged(w, pools, ent, sink=sink)
    compare(o, l, ro, rl, label=f"paged_uniform_H{H}_S{split}")


@pytest.mark.parametrize("H", [16, 64, 128])
def test_paged_persistent_grid(smla, H):
    """Enough ragged rows that the 16-head and wide-head kernels run one
    block per compute unit, each taking several units in turn, through both
    pools with sinks (empty rows among them): bit-identical to one unit per
    block, and the oracle's result on sampled rows."""
    rng = np.random.default_rng(95 + H)
    lens = rng.integers(0, 900, 400)
    lens[::11] = 0
    w = ragged_workload(f"paged_persist_H{H}", H, lens.tolist(), 12000, seed=96 + H, trailing=8)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(16, 8), pad=(3 * 656 + 16, 0))
    ent = entries(w, entry_of)
    sink = sink_values(rng, H)
    pools_d = to_dev(pools)
    note(f"paged persistent grid H={H} T={w.T}")
    o, l = run_paged(smla, w, pools_d, ent, sink=sink)
    smla.set_option("persist", 1)
    try:
        o1, l1 = run_paged(smla, w, pools_d, ent, sink=sink)
    finally:
        smla.set_option("persist", 0)
    assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l, l1)
    rows = sorted(set(sample_rows(w.T, 8, seed=H).tolist()) | {0, 11, w.T - 1})
    ro, rl = run_oracle_paged(w, pools, ent, sink=sink, rows=rows)
    compare(o, l, ro, rl, rows=rows, label=f"paged_persist_H{H}")


def test_paged_absent_pool(smla):
    """With the compressed pool absent, its entries are not keys: the result
    equals the oracle's with those entries replaced by -1, with and without
    has_invalid."""
    w = ragged_workload("paged_absent", 16, [900, 300, 2000], 4000, seed=80, invalid_p=0.0)
    rng = np.random.default_rng(81)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(32, 4), pad=(0, 0))
    ent = entries(w, entry_of)
    sink = rng.normal(0.0, 2.0, 16)
    ref_ent = np.where(ent < -1, -1, ent)
    ro, rl = run_oracle_paged(w, pools, ref_ent, sink=sink)
    pools_d = to_dev(pools)
    pools_d[1] = (None, 0, 0)
    for hi in (False, True):
        note(f"paged absent pool has_invalid={hi}")
        o, l = run_paged(smla, w, pools_d, ent, sink=sink, has_invalid=hi)
        compare(o, l, ro, rl, label=f"paged_absent_hi{int(hi)}")


def test_paged_all_entries_invalid(smla):
    """Rows whose every entry is -1 (or names the absent pool): out 0 and
    lse = sink (-inf where the sink is -inf), split or not."""
    T, H = 5, 16
    w = synth.build_workload("paged_none", T, H, 64,
                             lambda g, r, m: -np.ones(300 * r, np.int64), seed=82, has_invalid=1)
    rng = np.random.default_rng(83)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(8, 8), pad=(0, 0))
    ent = entries(w, entry_of)
    ent[1::2] = compressed_entry(5)        # a compressed slot of the absent pool
    pools_d = to_dev(pools)
    pools_d[1] = (None, 0, 0)
    sink = sink_values(rng, H)
    for split in (1, 4):
        note(f"paged all invalid split={split}")
        smla.set_option("split", split)
        try:
            o, l = run_paged(smla, w, pools_d, ent, sink=sink)
        finally:
            smla.set_option("split", 0)
        assert torch.all(o == 0)
        want = np.broadcast_to(sink.astype(np.float32), (T, H))
        np.testing.assert_allclose(l.cpu().numpy(), want, rtol=2e-6, atol=0)


def test_paged_pool_beyond_4gib(smla):
    """Compressed-pool pages far apart (page_stride 2 MiB + 64 records), so
    slots land more than 4 GiB past the pool's base: 64-bit page offsets."""
    rng = np.random.default_rng(84)
    T, H, k = 3, 16, 512
    w = synth.build_workload("paged_4g", T, H, 3000,
                             lambda g, r, m: synth.distinct_uniform(g, 3000, k), seed=85)
    kv = w.kv.numpy()
    per, stride = 64, 64 * 656 + (2 << 20)
    slots = rng.choice(2400 * per, kv.shape[0], replace=False).astype(np.int64)
    slots[:200] = 2400 * per - 1 - np.arange(200)   # the pool's far end
    offs = (slots // per) * stride + (slots % per) * 656
    nbytes = int(offs.max()) + 656
    assert nbytes > (4 << 30) + (64 << 20)
    note(f"paged pool beyond 4 GiB: {nbytes / 2**30:.2f} GiB")
    host = np.zeros(nbytes, np.uint8)              # untouched pages stay unbacked
    host[offs[:, None] + np.arange(656)[None, :]] = kv
    dev = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    dev[torch.from_numpy(offs[:, None] + np.arange(656)[None, :]).to(DEV)] = w.kv.to(DEV)
    win = (np.zeros(656, np.uint8), 656, 1)        # an unused one-record window pool
    pools = [win, (host, stride, per)]
    ent = compressed_entry(slots)[w.indices.numpy().astype(np.int64)]
    sink = rng.normal(0.0, 2.0, H)
    o, l = run_paged(smla, w, [(torch.from_numpy(win[0]).to(DEV), 656, 1), (dev, stride, per)],
                     ent, sink=sink)
    ro, rl = run_oracle_paged(w, pools, ent, sink=sink)
    del dev
    compare(o, l, ro, rl, label="paged_4g")


def test_paged_decode_full_size(smla):
    """The decode workload at full size (64 rows x 2048 keys of 65,536 records,
    16 heads) through two pools of 64-record pages with a sink, as the bench
    runs it: bit-identical to the contiguous forward without the sink, and
    sampled rows against the oracle with it."""
    w = synth.make_workload(2)
    rng = np.random.default_rng(86)
    pools, entry_of = paged_layout(rng, w.kv.numpy(), per_page=(64, 64), pad=(256, 0))
    ent = entries(w, entry_of)
    pools_d = to_dev(pools)
    note("paged decode full size, no sink")
    o_p, l_p = run_paged(smla, w, pools_d, ent)
    wd = w.to(DEV)
    o_c, l_c = smla.fwd(wd.q, wd.kv, wd.indptr, wd.indices, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))
    assert torch.equal(l_p, l_c)
    sink = rng.normal(0.0, 3.0, w.H)
    note("paged decode full size, sink")
    o, l = run_paged(smla, w, pools_d, ent, sink=sink)
    rows = sample_rows(w.T, 6, seed=87)
    ro, rl = run_oracle_paged(w, pools, ent, sink=sink, rows=rows)
    compare(o, l, ro, rl, rows=rows, label="paged_decode_full")
