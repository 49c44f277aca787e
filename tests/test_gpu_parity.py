"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name and shape before touching the GPU and its error
figures after.  Inputs are seeded and synthetic (synth/); the oracle never
sees anything the HIP path produced.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare, q_bits, run_gpu, run_oracle, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_fp8_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(autouse=True)
def _reset_split(smla):
    smla.set_option("split", 0)
    smla.set_option("persist", 0)
    yield
    smla.set_option("split", 0)
    smla.set_option("persist", 0)


def custom(name, H, N, slices, seed=11, device="cuda", **kw):
    slices = [np.asarray(s, dtype=np.int64) for s in slices]
    return synth.build_workload(name, len(slices), H, N, lambda g, r, m: slices[r],
                                seed=seed, device=device, **kw)


# ------------------------------------------------------------------ decode hook

def test_decode_rows_bitexact(smla):
    rng = np.random.default_rng(5)
    n = 512
    rec = np.zeros((n, 656), np.uint8)
    codes = np.tile(np.arange(256, dtype=np.uint8), (n, 2))
    codes = np.stack([rng.permutation(c) for c in codes])
    codes[(codes & 0x7F) == 0x7F] = 0x00  # the two NaN codes are covered separately
    rec[:, :512] = codes
    e = rng.integers(-22, 8, size=(n, 4)).astype(np.float64)
    sc = np.ldexp(1.0, e.astype(int)).astype("<f4")
    sc[::17, 2] = 0.0  # zero-scale blocks
    rec[:, 512:528] = sc.view(np.uint8).reshape(n, 16)
    rec[:, 528:] = rng.integers(0, 256, size=(n, 128), dtype=np.uint8)
    rec[:, 529::2] &= 0x7F ^ 0x40  # keep rope exponents finite
    kv = torch.from_numpy(rec).to(DEV)
    rows = torch.from_numpy(np.concatenate([rng.permutation(n), [-1, n]]).astype(np.int32)).to(DEV)
    note(f"decode_rows n={n}")
    got = smla.decode_rows(kv, rows).cpu().numpy()
    ref = oracle.decode_records(rec[rows.cpu().numpy()[:n]]).astype(np.float32)
    # zero-scale blocks: the QK conversion applies the scale's exponent field,
    # so they decode to code * 2^-127 (a zero latent for attention purposes)
    zmask = np.zeros((n, 576), bool)
    zrow = np.isin(rows.cpu().numpy()[:n], np.arange(0, n, 17))
    zmask[np.ix_(zrow, np.arange(256, 384))] = True
    assert np.all(np.abs(got[:n][zmask]) <= 2.0 ** -118)
    gb, rb = got[:n].view(np.uint32), ref.view(np.uint32)
    bad = np.argwhere((gb != rb) & ~zmask)
    detail = [(int(i), int(j), float(got[i, j]), float(ref[i, j]), hex(int(rec[rows.cpu().numpy()[i], j])) if j < 512 else "rope")
              for i, j in bad[:12]]
    assert bad.size == 0, f"{len(bad)} mismatching values, first: {detail}"
    assert np.all(np.isnan(got[n:]))


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(smla, cfg):
    c = synth.make_config(cfg)
    note(f"config {cfg} {c['name']} T={c['T']} H={c['H']} N={c['N']}")
    w = synth.make_workload(cfg, device="cuda")
    out, lse = run_gpu(w)
    rows = None if cfg != 5 else stratified_rows(w.T)
    if cfg == 3:
        ro, rl, ra = run_oracle(w, rows=rows, with_abs=True)
        st = compare(out, lse, ro, rl, rows=rows, large_values=True, abs_ref=ra, label=f"config{cfg}")
    else:
        ro, rl = run_oracle(w, rows=rows)
        st = compare(out, lse, ro, rl, rows=rows, label=f"config{cfg}")
    print(f"config {cfg}: {len(rows) if rows is not None else w.T} rows checked; {st}")


def stratified_rows(T):
    """512 rows spread over the batch and over the eight XCD slots (a row's
    rank mod 8): row 64k + 8j + (k + j) mod 8 for k < T/64, j < 8, plus the
    last row."""
    rows = [64 * k + 8 * j + (k + j) % 8 for k in range(T // 64) for j in range(8)]
    return np.unique(np.array(rows + [T - 1], dtype=np.int64))


# ------------------------------------------------------------------ edge cases

def edge_slices(N, rng):
    s = [
        [],                                   # empty
        [-1, -1, -1],                          # all invalid
        [int(rng.integers(N))],                # single key
        rng.integers(0, N, 31).tolist(),       # < one wave's 32
        rng.integers(0, N, 33).tolist(),       # crosses a wave boundary
        rng.integers(0, N, 127).tolist(),      # ragged tail
        rng.integers(0, N, 129).tolist(),      # one past a 128-token tile
        rng.integers(0, N, 300).tolist() + [-1] * 70,            # trailing padding
        [-1] * 40 + rng.integers(0, N, 50).tolist() + [-1] * 9,  # leading and trailing -1
        (rng.integers(0, N, 200) * (rng.random(200) < 0.7) - (rng.random(200) >= 0.7)).tolist(),
        rng.integers(0, N, 1000).tolist(),
        [int(N - 1)] * 5,                      # duplicates of the last row
    ]
    return s


@pytest.mark.parametrize("has_invalid", [0, 1])
def test_edge_rows(smla, has_invalid):
    rng = np.random.default_rng(21)
    N = 5000
    w = custom("edges", 16, N, edge_slices(N, rng), has_invalid=has_invalid)
    note(f"edge rows has_invalid={has_invalid} T={w.T}")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label=f"edges_inv{has_invalid}")


def test_negative_length_rows(smla):
    rng = np.random.default_rng(22)
    w = custom("neglen", 16, 600, [rng.integers(0, 600, 50), rng.integers(0, 600, 70), rng.integers(0, 600, 40)])
    ip = w.indptr.cpu().numpy()
    ip[1] = ip[2] + 5  # row 0 grows past row 1's end, row 1 gets a negative length
    w.indptr = torch.from_numpy(ip).to(DEV)
    note("negative length")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    assert np.isneginf(rl[1]).all()
    compare(out, lse, ro, rl, label="neglen")


@pytest.mark.parametrize("H", [1, 7, 16, 17, 32, 33, 48, 64, 65, 96, 100, 128])
def test_head_counts(smla, H):
    rng = np.random.default_rng(100 + H)
    N = 3000
    sl = [rng.integers(0, N, int(L)) for L in rng.integers(0, 400, 9)]
    w = custom(f"heads{H}", H, N, sl, seed=H)
    note(f"H={H} T={w.T}")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label=f"H{H}")


@pytest.mark.parametrize("has_invalid,split,outliers", [(0, 1, 0), (1, 1, 0), (0, 3, 0), (1, 2, 1), (0, 1, 1)])
def test_wide_stream_edges(smla, has_invalid, split, outliers):
    """Above 32 heads each score wave takes one half of a 32-token tile, and
    the two halves (tokens 0-15 and 16-31) are two softmax streams with their
    own references, merged by powers of two.  Rows here end inside, on and
    just past a half or a tile, have one half of every tile masked, or carry
    outlier latents (large logits: the references move, O and the sums are
    rescaled)."""
    rng = np.random.default_rng(31 + 4 * has_invalid + split + 8 * outliers)
    N = 4000
    sl = [rng.integers(0, N, L) for L in (1, 5, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 700)]
    pos = np.arange(160) % 32
    x = rng.integers(0, N, 160)
    x[pos >= 16] = -1  # the second half of every tile masked
    y = rng.integers(0, N, 160)
    y[pos < 16] = -1   # the first half masked
    z = rng.integers(0, N, 160)
    z[pos != 20] = -1  # one key per tile, in the second half
    sl += [x, y, z]
    kw = dict(latent_std=2.0, outlier_p=0.01, outlier_mag=1000.0) if outliers else {}
    w = custom(f"streams_inv{has_invalid}_s{split}_o{outliers}", 64, N, sl, seed=50 + split, has_invalid=has_invalid, **kw)
    smla.set_option("split", split)
    note(f"wide stream edges has_invalid={has_invalid} split={split} outliers={outliers} T={w.T}")
    out, lse = run_gpu(w)
    if outliers:  # outputs near 10^3: the per-element bound of the ragged workload (reading c14)
        ro, rl, ra = run_oracle(w, with_abs=True)
        compare(out, lse, ro, rl, large_values=True, abs_ref=ra, label=f"streams inv{has_invalid} s{split} o1")
    else:
        ro, rl = run_oracle(w)
        compare(out, lse, ro, rl, label=f"streams inv{has_invalid} s{split} o0")


@pytest.mark.parametrize("H,split,has_invalid", [(16, 0, 0), (16, 2, 1), (64, 0, 0), (64, 3, 0), (64, 2, 1), (128, 2, 0)])
def test_guessed_slice_starts(smla, H, split, has_invalid):
    """Without a plan and with nnz a multiple of T, each unit guesses its slice
    start (row x nnz/T) and queues its first index tiles before indptr
    arrives.  The rows here make the guess right for some units and wrong for
    others (the start, the length or a chunk's bounds differ; one row is
    empty), so both the kept and the re-queued index tiles are checked."""
    rng = np.random.default_rng(60 + H + split + has_invalid)
    N = 5000
    lengths = [300, 100, 200, 200, 0, 400, 200, 200]  # nnz = 1,600 = 8 x 200
    sl = [rng.integers(0, N, L) for L in lengths]
    if has_invalid:  # trailing and interior padding inside the same lengths
        sl[2][150:] = -1
        sl[3][::7] = -1
        sl[6][:] = -1
    w = custom(f"guess_H{H}_s{split}_inv{has_invalid}", H, N, sl, seed=61 + H, has_invalid=has_invalid)
    assert w.nnz % w.T == 0
    smla.set_option("split", split)
    note(f"guessed slice starts H={H} split={split} has_invalid={has_invalid} T={w.T}")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label=f"guess H{H} s{split} inv{has_invalid}")


@pytest.mark.parametrize("split", [1, 2, 3, 7, 32])
def test_forced_split(smla, split):
    rng = np.random.default_rng(7)
    N = 20000
    sl = [rng.integers(0, N, int(L)) for L in (2048, 1, 700, 0, 1500, 129)]
    w = custom("split", 16, N, sl)
    smla.set_option("split", split)
    note(f"split={split}")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label=f"split{split}")


@pytest.mark.parametrize("split,H", [(2, 16), (3, 7), (4, 16), (8, 16), (8, 1), (3, 64), (2, 128), (5, 40)])
def test_split_merge_back_to_back(smla, split, H):
    """Split rows: several forwards queued back to back on one stream (new
    inputs each time) must each match the oracle, so the partials of one call
    never leak into the next."""
    rng = np.random.default_rng(20 + split)
    N = 9000
    ws = []
    for k in range(4):
        sl = [rng.integers(0, N, int(L)) for L in (1024, 0, 1, 513, 1024, 97, 300)]
        ws.append(custom(f"b2b{k}", H, N, sl, seed=100 + k))
    smla.set_option("split", split)
    note(f"back-to-back split={split} H={H}")
    outs = []
    for w in ws:
        outs.append(smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale))
    torch.cuda.synchronize()
    for k, (w, (out, lse)) in enumerate(zip(ws, outs)):
        ro, rl = run_oracle(w)
        compare(out, lse, ro, rl, label=f"b2b{k} split{split} H{H}")


@pytest.mark.parametrize("H", [16, 64])
def test_long_rows_max_split(smla, H):
    """Two rows of 65,536 keys each (512 tiles of 128 / 1024 of 64): the
    automatic split reaches its cap of 32 chunks, and the combine merges 32
    partials per row; plus a one-key row in between."""
    rng = np.random.default_rng(40 + H)
    N = 65536
    sl = [rng.permutation(N), np.array([N - 1]), rng.permutation(N)]
    w = custom(f"long_rows_H{H}", H, N, sl, seed=41 + H)
    assert smla.split_for(w.T, w.H, w.nnz) == 32
    note(f"long rows H={H} nnz={w.nnz}")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label=f"long_rows_H{H}")


def test_workspace_reuse_across_shapes(smla):
    """One uninitialised workspace serves a split forward, a larger unsplit one
    and the split one again."""
    rng = np.random.default_rng(31)
    N = 5000
    small = custom("reuse_small", 16, N, [rng.integers(0, N, 900) for _ in range(5)])
    big = custom("reuse_big", 16, N, [rng.integers(0, N, 200) for _ in range(300)], seed=12)
    ws = torch.empty(max(smla.workspace_bytes(5, 16, small.nnz), smla.workspace_bytes(300, 16, big.nnz)),
                     dtype=torch.uint8, device=DEV)
    note("workspace reuse across shapes")
    res = []
    for w in (small, big, small):
        res.append(smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, ws=ws))
    torch.cuda.synchronize()
    for w, (out, lse) in zip((small, big, small), res):
        ro, rl = run_oracle(w)
        compare(out, lse, ro, rl, label=w.name)


def test_single_index_is_exact(smla):
    rng = np.random.default_rng(8)
    N = 700
    w = custom("single", 16, N, [[int(i)] for i in rng.integers(0, N, 40)])
    note("single index per row")
    out, lse = run_gpu(w)
    K = oracle.decode_records(w.kv.cpu().numpy()[w.indices.cpu().numpy()])
    want = torch.from_numpy(K[:, :512]).float().to(torch.bfloat16)[:, None, :].expand(-1, 16, -1)
    assert torch.equal(out.cpu(), want), "one key must return that record's latent exactly"
    Q = oracle.bf16_bits_to_f64(q_bits(w))
    s = w.sm_scale * np.einsum("thd,td->th", Q, K)
    assert np.max(np.abs(lse.cpu().numpy() - s)) <= 1e-3


def test_strided_q_out_and_no_lse(smla):
    rng = np.random.default_rng(9)
    N = 4000
    sl = [rng.integers(0, N, int(L)) for L in (300, 5, 640)]
    w = custom("strided", 16, N, sl)
    qbig = torch.zeros(w.T, 19, 584, dtype=torch.bfloat16, device=DEV)
    qbig[:, 2:18, :576] = w.q.to(DEV)
    obig = torch.full((w.T, 20, 520), 7.0, dtype=torch.bfloat16, device=DEV)
    note("strided q/out, no lse")
    out, lse = run_gpu(w, q=qbig[:, 2:18, :576], out=obig[:, 3:19, :512], return_lse=False)
    assert lse is None
    ro, rl = run_oracle(w)
    compare(out, None, ro, rl, label="strided")
    assert torch.all(obig[:, :3] == 7.0) and torch.all(obig[:, 19:] == 7.0)
    assert torch.all(obig[:, :, 512:] == 7.0)


def test_empty_index_stream(smla):
    w = custom("nnz0", 16, 10, [[], [], []])
    note("nnz = 0")
    out, lse = run_gpu(w)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_zero_scale_records(smla):
    rng = np.random.default_rng(12)
    N = 300
    w = custom("zeroscale", 16, N, [rng.integers(0, N, 200), rng.integers(0, N, 33)])
    kv = w.kv.cpu().numpy()
    kv[::3, 512:528] = 0  # every third record: all four scales zero
    kv[1::3, 516:520] = 0  # block 1 zero
    w.kv = torch.from_numpy(kv).to(DEV)
    note("zero-scale records")
    out, lse = run_gpu(w)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label="zeroscale")


def test_permutation_duplicates(smla):
    rng = np.random.default_rng(13)
    N = 2500
    base = [rng.integers(0, N, 500), rng.integers(0, N, 77)]
    w1 = custom("perm_a", 16, N, base, seed=3)
    w2 = custom("perm_b", 16, N, [rng.permutation(b) for b in base], seed=3)
    w3 = custom("dups", 16, N, [np.repeat(b, 2) for b in base], seed=3)
    note("permutation / duplicates")
    o1, l1 = run_gpu(w1)
    o2, l2 = run_gpu(w2)
    o3, l3 = run_gpu(w3)
    ro, rl = run_oracle(w1)
    compare(o2, l2, ro, rl, label="permuted")
    compare(o3, l3 - math.log(2), ro, rl, label="duplicated")


@pytest.mark.parametrize("H", [16, 64, 128])
def test_causal_ragged_longest_first(smla, H):
    """Many ragged rows (row r has min(3r + 1, 2048) keys): exercises the
    longest-first order and has_invalid trimming at scale (above 64 heads,
    with two head groups per row)."""
    T, N = 600, 32768
    rng = np.random.default_rng(14)
    sl = []
    for r in range(T):
        L = min(3 * r + 1, 2048)
        sl.append(np.concatenate([rng.integers(0, N, L), -np.ones(2048 - L, np.int64)]))
    w = custom(f"causal_H{H}", H, N, sl, has_invalid=1)
    note(f"causal ragged T={T} H={H}")
    out, lse = run_gpu(w)
    rows = sample_rows(T, 40 if H == 16 else 12, seed=1)
    ro, rl = run_oracle(w, rows=rows)
    compare(out, lse, ro, rl, rows=rows, label=f"causal_H{H}")


def test_ragged_causal_prefill_workload(smla):
    """The additional workload: a 2,048-token causal prefill at 64 heads (row r
    attends to tokens 0 .. r, padded to 2,048 with -1), every row computed and
    sampled rows against the oracle, the first row (one key) and the last (all
    2,048) among them."""
    w = synth.make_workload(6, device="cuda")
    note(f"ragged causal prefill {w.name}")
    out, lse = run_gpu(w)
    rows = sorted(set(sample_rows(w.T, 16, seed=6).tolist()) | {1, 31, 32, 33})
    ro, rl = run_oracle(w, rows=rows)
    compare(out, lse, ro, rl, rows=rows, label="ragged_causal_prefill")


@pytest.mark.parametrize("H,split,T", [(64, 0, 700), (128, 0, 700), (40, 0, 700), (64, 2, 700),
                                       (16, 0, 240), (16, 2, 240), (5, 3, 160)])
def test_persistent_grid(smla, H, split, T):
    """Ragged rows, many more units than compute units, so that the 16-head and
    wide-head kernels run one block per compute unit, each block taking
    several units in turn.  Empty rows and rows of every length sit between
    long ones, so blocks pass from empty units to full ones and back.  The
    result is bit-identical to one unit per block (each unit's arithmetic does
    not depend on the block that runs it) and matches the oracle on sampled
    rows, the empty ones among them.  (The 16-head kernel takes the persistent
    grid only up to two units per CU, hence fewer rows there.)"""
    N = 40000
    rng = np.random.default_rng(20 + H + split)
    lens = rng.integers(0, 1300, T)
    lens[::9] = 0
    lens[5::13] = 1
    lens[7::31] = 2048
    sl = [np.where(rng.random(L) < 0.03, -1, rng.integers(0, N, L)) for L in lens]
    w = custom(f"persist_H{H}_S{split}", H, N, sl, seed=21, has_invalid=1)
    note(f"persistent grid T={T} H={H} split={split}")
    smla.set_option("split", split)
    out, lse = run_gpu(w)
    smla.set_option("persist", 1)
    out1, lse1 = run_gpu(w)
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse, lse1)
    rows = sorted(set(sample_rows(T, 10, seed=H).tolist()) | {0, 5, 7, 9, T - 1})
    ro, rl = run_oracle(w, rows=rows)
    compare(out, lse, ro, rl, rows=rows, label=f"persist_H{H}_S{split}")


def test_repeat_calls_bitwise_identical(smla):
    w = synth.make_workload(2, device="cuda", T=16)
    note("repeat determinism")
    o1, l1 = run_gpu(w)
    o2, l2 = run_gpu(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_scale_above_cap_stays_finite(smla):
    """A scale above 2^7 breaks a precondition: the result must stay finite."""
    rng = np.random.default_rng(15)
    N = 200
    w = custom("bigscale", 16, N, [rng.integers(0, N, 100)])
    kv = w.kv.cpu().numpy()
    kv[:, 512:516] = np.frombuffer(np.float32(2.0 ** 10).tobytes(), np.uint8)
    w.kv = torch.from_numpy(kv).to(DEV)
    note("scale above cap")
    out, lse = run_gpu(w)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
