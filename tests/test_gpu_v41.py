"""GPU parity of the V4.1 key record path (sparse_mla_fwd_v41 and the MXFP8
test hook, through the C ABI) against the fp64 oracle (oracle.v41).

* The MXFP8 quantiser (the combine's own device code, through
  sparse_mla_mxfp8) must give the oracle's codes and scale bytes bit for bit
  on the same f32 values: the rounding decisions are taken on identical
  inputs.
* The forward + epilogue is compared where floating point allows: lse within
  1e-3; the values the epilogue quantises (y: bf16 output, rope dims rotated
  back) against the oracle's y with the attention tolerances plus one bf16
  step (both sides round their own f32/f64 result to bf16); the MXFP8 output
  must be the quantisation of the GPU's own y (within half an E4M3 step, or
  the saturation of the block's top binade) and its scale bytes must be those
  of the GPU's y blocks; where the oracle's block maximum is not within 2%
  of a power of two, the scale bytes must equal the oracle's.

Inputs are seeded and synthetic (synth.v41); every case prints its name
before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.v41 as ov
import synth.v41 as sv
from pools import v41_layout

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
OUT_REL_L2 = 1e-2
OUT_ABS = 3e-2
LSE_ABS = 1e-3


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_fp8_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield m
    m.set_option("split", 0)


# ----------------------------------------------------------------- MXFP8 hook

def mx_inputs(rng, nblocks):
    """f32 values in 32-blocks: N(0,1) at random magnitudes 2^-140 .. 2^100,
    plus blocks of zeros, -0.0, exact powers of two, midpoints of E4M3 codes
    (ties), values that saturate, f32 subnormals and blocks just below a
    power of two."""
    y = rng.standard_normal((nblocks, 32)) * np.exp2(rng.uniform(-140, 100, (nblocks, 1)))
    y[0] = 0.0
    y[1] = -0.0
    y[2] = np.exp2(rng.integers(-20, 20, 32)).astype(np.float64)
    codes = np.arange(0x40, 0x5F)
    mids = (oracle.E4M3_TABLE[codes] + oracle.E4M3_TABLE[codes + 1]) / 2
    y[3, 0] = 256.0
    y[3, 1:] = mids[:31] * rng.choice([-1.0, 1.0], 31)
    y[4] = rng.uniform(448.0, 511.9, 32) * rng.choice([-1.0, 1.0], 32)     # E = 0, most saturate
    y[5] = rng.standard_normal(32) * 2.0 ** -140                        # f32 subnormals
    y[6] = (2.0 - 2.0 ** -20) * rng.choice([-1.0, 1.0], 32)             # just below 2
    y[7, :] = 1.0
    y[7, 5] = -0.0
    y[7, 6] = 1e-6                                                      # rounds to +0 at this scale
    y[7, 7] = -1e-6                                                     # rounds to -0
    return y.astype(np.float32)


def test_mxfp8_hook_bitexact(smla):
    rng = np.random.default_rng(90)
    y = mx_inputs(rng, 4096)                                            # 131072 values
    note(f"mxfp8 hook n={y.size}")
    codes, scales = smla.mxfp8(torch.from_numpy(y.reshape(-1)).to(DEV))
    torch.cuda.synchronize()
    want_c, want_s = ov.mxfp8_quantize(y.astype(np.float64).reshape(-1))
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.flatnonzero(got_s != want_s)
    assert bad.size == 0, f"{bad.size} scale bytes differ, first block {bad[0]}: {got_s[bad[0]]} vs {want_s[bad[0]]}"
    bad = np.flatnonzero(got_c != want_c)
    assert bad.size == 0, (f"{bad.size} codes differ, first {bad[0]}: y={y.reshape(-1)[bad[0]]!r} "
                           f"got {got_c[bad[0]]:#x} want {want_c[bad[0]]:#x}")


# ----------------------------------------------------------------- forward + epilogue

class Case:
    pass


def make_case(T, H, N, lens, seed, per_page=(32, 16), pad=(32, 0), invalid_p=0.03, trailing=0,
              sink=None, n_pos=4096, sigma=1.0, outlier_p=0.0):
    rng = np.random.default_rng(seed)
    c = Case()
    c.data, c.scales = sv.make_v41_keys(N, seed=seed, sigma=sigma, outlier_p=outlier_p)
    c.pools, entry_of = v41_layout(rng, c.data, c.scales, per_page=per_page, pad=pad)
    sl = []
    for L in lens:
        e = entry_of[rng.permutation(N)[:L]] if L else np.zeros(0, np.int64)
        if L and invalid_p > 0:
            e = np.where(rng.random(L) < invalid_p, -1, e)
        sl.append(np.concatenate([e, -np.ones(trailing, np.int64)]))
    c.indptr = np.concatenate([[0], np.cumsum([len(s) for s in sl])]).astype(np.int32)
    c.indices = (np.concatenate(sl) if sl else np.zeros(0)).astype(np.int32)
    c.q = sv.make_q(T, H, seed=seed + 1)
    c.cos_sin = sv.make_cos_sin(n_pos)
    c.pos = rng.integers(0, n_pos, T).astype(np.int32)
    c.sink = sink
    c.sm_scale = sv.sm_scale_v41()
    c.has_invalid = bool(invalid_p > 0 or trailing > 0)
    c.T, c.H = T, H
    return c


def run_gpu(smla, c, pos=None, q_dev=None):
    pools_d = [(torch.from_numpy(b).to(DEV), st, pr) for b, st, pr in c.pools]
    sk = None if c.sink is None else torch.from_numpy(np.asarray(c.sink, np.float32)).to(DEV)
    xo, xos, lse, y = smla.fwd_v41(
        c.q.to(DEV) if q_dev is None else q_dev, pools_d, torch.from_numpy(c.indptr).to(DEV), torch.from_numpy(c.indices).to(DEV),
        c.sm_scale, torch.from_numpy(c.pos if pos is None else pos).to(DEV),
        torch.from_numpy(c.cos_sin).to(DEV), sink=sk, has_invalid=c.has_invalid, return_y=True)
    torch.cuda.synchronize()
    return xo.cpu().numpy(), xos.cpu().numpy(), lse.cpu().numpy().astype(np.float64), \
        y.cpu().numpy().astype(np.float64)


def run_oracle(c, rows=None):
    qb = c.q.view(torch.int16).numpy().view(np.uint16)
    out, lse = ov.sparse_mla_fwd_v41(qb, c.pools, c.indptr, c.indices, c.sm_scale,
                                     sink=None if c.sink is None else np.asarray(c.sink, np.float64), rows=rows)
    rr = np.arange(c.T) if rows is None else np.asarray(rows)
    y = np.full_like(out, np.nan)
    y[rr], _, _ = ov.v41_epilogue(out[rr], c.cos_sin, c.pos[rr])
    return y, lse


def check(c, got, want, rows=None, label=""):
    xo, xos, lse_g, y_g = got
    y_o, lse_o = want
    rr = np.arange(c.T) if rows is None else np.asarray(rows)
    xo, xos, lse_g, y_g, y_o, lse_o = xo[rr], xos[rr], lse_g[rr], y_g[rr], y_o[rr], lse_o[rr]
    stats = {}
    # lse: -inf where the oracle has no key and no sink, else within 1e-3
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isneginf(lse_g), ~fin), f"{label}: -inf lse positions differ"
    if fin.any():
        stats["lse_max_abs"] = float(np.max(np.abs(lse_g[fin] - lse_o[fin])))
        assert stats["lse_max_abs"] <= LSE_ABS, f"{label}: lse {stats['lse_max_abs']}"
    # y: attention tolerances plus one bf16 step of each side's rounding
    d = y_g - y_o
    nr = np.linalg.norm(y_o)
    stats["y_rel_l2"] = float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d))
    stats["y_max_abs"] = float(np.max(np.abs(d)))
    assert stats["y_rel_l2"] <= OUT_REL_L2, f"{label}: y rel L2 {stats['y_rel_l2']}"
    worst = np.max(np.abs(d) - (OUT_ABS + 2.0 ** -7 * np.abs(y_o)))
    assert worst <= 0, f"{label}: y max abs {stats['y_max_abs']} over the bound by {worst}"
    # the MXFP8 output is the quantisation of the GPU's own y: each block's
    # scale 2^E puts its largest magnitude in [256, 512) (E = -127 below that)
    E = xos.astype(np.int64) - 127
    blk_amax = np.abs(y_g.reshape(y_g.shape[:-1] + (16, 32))).max(axis=-1)
    r = blk_amax * np.exp2(-E.astype(np.float64))
    ok_e = ((r >= 256.0) & (r < 512.0)) | ((E == -127) & (r < 512.0))
    assert np.all(ok_e), f"{label}: scale bytes are not those of y's blocks"
    dq = ov.mxfp8_dequantize(xo, xos)
    scale = np.repeat(np.exp2(E), 32, axis=-1)
    step = np.maximum(np.abs(y_g) * 2.0 ** -4, scale * 2.0 ** -10)
    excess = np.maximum(np.abs(y_g) - 448.0 * scale, 0.0)
    assert np.all(np.abs(dq - y_g) <= step + excess), f"{label}: MXFP8 codes are not y's quantisation"
    # and, where the block maximum is not near a power of two, the oracle's scale bytes
    o_amax = np.abs(y_o.reshape(y_o.shape[:-1] + (16, 32))).max(axis=-1)
    with np.errstate(divide="ignore"):
        frac = np.abs(np.log2(np.where(o_amax > 0, o_amax, 1.0)) - np.round(np.log2(np.where(o_amax > 0, o_amax, 1.0))))
    clear = (frac > np.log2(1.02)) | (o_amax == 0)
    want_e = ov.mx_exponent(o_amax)
    assert np.array_equal(E[clear], want_e[clear]), f"{label}: scale bytes differ from the oracle's"
    print(f"[parity] {label} {stats}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("H", [16, 5, 1])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_v41_matches_oracle(smla, H, split):
    """Both pools, scattered -1 entries, trailing padding, an empty row, a
    one-key row and rows across several 128-key tiles; per-head sinks."""
    rng = np.random.default_rng(91 + H)
    sink = rng.normal(0.0, 2.0, H)
    sink[0] = -np.inf
    lens = [0, 1, 127, 129, 700, 2048, 333]
    c = make_case(len(lens), H, 6000, lens, seed=92 + H + split, trailing=20, sink=sink)
    note(f"v41 H={H} split={split}")
    smla.set_option("split", split)
    try:
        got = run_gpu(smla, c)
    finally:
        smla.set_option("split", 0)
    check(c, got, run_oracle(c), label=f"v41_H{H}_S{split}")
    xo, xos, lse, y = got
    # the empty row: y = 0 (rotated zeros may carry a sign: E4M3 +-0), scale byte 0
    assert np.all((xo[0] & 0x7F) == 0) and np.all(xos[0] == 0)
    np.testing.assert_allclose(lse[0], np.asarray(sink, np.float32), rtol=2e-6, atol=0)


def test_v41_no_sink_all_invalid_and_outliers(smla):
    """No sink (lse -inf for keyless rows), a row of -1 only, and latent
    outliers of +-1000 with scale bytes up to 2^2 per block."""
    lens = [300, 0, 1500, 64]
    c = make_case(len(lens), 16, 4000, lens, seed=93, sigma=2.0, outlier_p=0.01)
    c.indices[c.indptr[0]:c.indptr[1]] = -1
    note("v41 no sink, outliers")
    got = run_gpu(smla, c)
    check(c, got, run_oracle(c), label="v41_outliers")
    assert np.all(np.isneginf(got[2][0])) and np.all((got[0][0] & 0x7F) == 0)


def test_v41_position_clamped(smla):
    """Positions past the cos/sin table read its last row (memory-safe clamp)."""
    c = make_case(3, 16, 2000, [500, 20, 900], seed=94, n_pos=64)
    note("v41 position clamp")
    base = run_gpu(smla, c, pos=np.array([63, 63, 0], np.int32))
    clamped = run_gpu(smla, c, pos=np.array([63, 5000, -7], np.int32))
    for a, b in zip(base, clamped):
        assert np.array_equal(a, b)


def test_v41_strided_q(smla):
    """q as a strided device view (head pitch 520 elements, row pitch 19
    heads, starting one head in): the same bytes out as the contiguous q."""
    c = make_case(5, 16, 3000, [700, 1, 300, 2048, 129], seed=97)
    note("v41 strided q")
    base = run_gpu(smla, c)
    big = torch.zeros(c.T, c.H + 3, 520, dtype=torch.bfloat16, device=DEV)
    big[:, 1:c.H + 1, :512] = c.q.to(DEV)
    qv = big[:, 1:c.H + 1, :512]
    assert qv.stride() == ((c.H + 3) * 520, 520, 1)
    strided = run_gpu(smla, c, q_dev=qv)
    for a, b in zip(base, strided):
        assert np.array_equal(a, b, equal_nan=True)


def test_v41_decode_full_size(smla):
    """Decode shape of a V4.1 layer's rank: 64 rows x 16 heads x 2,048 keys of
    65,536 (64-key pages in both pools); sampled rows against the oracle."""
    T, H, N, k = 64, 16, 65536, 2048
    rng = np.random.default_rng(95)
    sink = rng.normal(0.0, 2.0, H)
    c = make_case(T, H, N, [k] * T, seed=96, per_page=(64, 64), pad=(0, 0), invalid_p=0.0, sink=sink)
    note("v41 decode full size")
    got = run_gpu(smla, c)
    rows = np.array([0, 17, 31, 40, 58, 63])
    check(c, got, run_oracle(c, rows=rows), rows=rows, label="v41_full")
