"""Pins for the CPU oracle (no GPU).

Each pin ties the oracle to something other than itself: the OCP E4M3 table
and torch's float8/bfloat16 casts (library), hand-decoded records, the
FlyDSL page's writer bound, pure-Python brute force on tiny inputs, torch's
scaled_dot_product_attention on the dense special case, and closed-form
invariants.  ``test_planted_mistakes`` plants plausible errors in the oracle
(on the CPU) and checks that some pin catches every one of them.
"""

import math
import struct

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
import oracle.codec as ocodec
import synth
from pools import paged_layout

SIGMA = float(np.float32(1.0 / math.sqrt(576)))


# ----------------------------------------------------------------- helpers

def random_records(rng, n, scale_exp=(-22, 7)):
    """Random but valid records: any non-NaN e4m3 code, pow2 scales, finite bf16 rope."""
    rec = np.zeros((n, 656), np.uint8)
    codes = rng.integers(0, 256, size=(n, 512))
    codes[(codes & 0x7F) == 0x7F] = 0x38
    rec[:, :512] = codes
    e = rng.integers(scale_exp[0], scale_exp[1] + 1, size=(n, 4))
    rec[:, 512:528] = np.ldexp(1.0, e).astype("<f4").view(np.uint8).reshape(n, 16)
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    rec[:, 528:] = torch.from_numpy(rope).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint8).reshape(n, 128)
    return rec


def random_q(rng, T, H, std=1.0):
    x = torch.from_numpy(rng.standard_normal((T, H, 576)) * std).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def torch_decode(rec):
    """Independent record decode through torch's own float8 / bfloat16 casts."""
    rec = np.ascontiguousarray(rec)
    n = rec.shape[0]
    lat = torch.from_numpy(rec[:, :512].copy()).view(torch.float8_e4m3fn).double().numpy()
    sc = np.frombuffer(rec[:, 512:528].tobytes(), dtype="<f4").reshape(n, 4).astype(np.float64)
    rope = torch.from_numpy(rec[:, 528:].copy()).view(torch.bfloat16).double().numpy()
    return np.concatenate([lat * np.repeat(sc, 128, axis=1), rope], axis=1)


def torch_q(q_bits):
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def brute_force(q_bits, kv, indptr, indices, sigma):
    """Pure-Python loops (math.fsum / math.exp) over torch-decoded inputs."""
    T, H, _ = q_bits.shape
    Q = torch_q(q_bits)
    out = np.zeros((T, H, 512))
    lse = np.full((T, H), -np.inf)
    for r in range(T):
        keys = [int(i) for i in indices[indptr[r]:indptr[r + 1]] if i >= 0] \
            if indptr[r + 1] > indptr[r] else []
        if not keys:
            continue
        K = torch_decode(kv[keys])
        for h in range(H):
            s = [sigma * math.fsum(float(a) * float(b) for a, b in zip(Q[r, h], K[j]))
                 for j in range(len(keys))]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = math.fsum(p)
            for d in range(512):
                out[r, h, d] = math.fsum(p[j] * K[j, d] for j in range(len(keys))) / l
            lse[r, h] = m + math.log(l)
    return out, lse


def tiny_case(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 5))
    H = int(rng.integers(1, 4))
    N = int(rng.integers(1, 17))
    kv = random_records(rng, N)
    q = random_q(rng, T, H, std=float(rng.choice([0.5, 1.0, 3.0])))
    slices = []
    for _ in range(T):
        L = int(rng.integers(0, 11))
        s = rng.integers(-1, N, size=L)  # -1 entries and duplicates allowed
        slices.append(s)
    indptr = np.zeros(T + 1, np.int64)
    indptr[1:] = np.cumsum([s.size for s in slices])
    idx = np.concatenate(slices).astype(np.int64) if slices else np.zeros(0, np.int64)
    return q, kv, indptr, idx


def assert_close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    if fin.any():
        assert np.max(np.abs(a[fin] - b[fin])) <= tol * max(1.0, np.max(np.abs(b[fin])))


# ----------------------------------------------------------------- codec pins

def test_e4m3_table_matches_torch():
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = ocodec.E4M3_TABLE
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_e4m3_spec_points(golden):
    for code, val in golden("e4m3_points.txt"):
        c = int(code, 16)
        v = float(val)
        got = ocodec.e4m3_value(c)
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), (code, got, v)


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    got = ocodec.bf16_bits_to_f64(bits)
    want = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_handbuilt_record(golden):
    rec = np.zeros((1, 656), np.uint8)
    rec[0, 512:528] = np.frombuffer(struct.pack("<4f", 2.0 ** -3, 2.0 ** 5, 1.0, 4.0), np.uint8)
    want = {}
    for pos, byte, blk, val in golden("handbuilt_record.txt"):
        pos, b = int(pos), int(byte, 16)
        if blk == "rope":
            off = 528 + 2 * (pos - 512)
            rec[0, off], rec[0, off + 1] = b & 0xFF, b >> 8
        else:
            assert int(blk) == pos // 128
            rec[0, pos] = b
        want[pos] = float(val)
    K = oracle.decode_records(rec)[0]
    for pos, val in want.items():
        assert K[pos] == val, (pos, K[pos], val)
    zero = [i for i in range(576) if i not in want]
    assert np.all(K[zero] == 0.0)


def test_record_decode_matches_torch():
    rec = random_records(np.random.default_rng(1), 64)
    assert np.array_equal(oracle.decode_records(rec), torch_decode(rec))


def test_writer_bound(golden):
    """The generator's writer meets the page's bound: scale 2^7 iff |latent| <= 57344."""
    for amax, scale in golden("writer_bound.txt"):
        amax, scale = float(amax), float(scale)
        lat = torch.zeros(1, 512)
        lat[0, :128] = amax
        rec = synth.encode_records(lat, torch.zeros(1, 64)).numpy()
        K = oracle.decode_records(rec)[0]
        assert np.frombuffer(rec[0, 512:516].tobytes(), "<f4")[0] == scale
        assert K[0] == amax  # exactly representable at that scale
    lat = torch.zeros(1, 512)
    lat[0, 0] = 57345.0
    rec = synth.encode_records(lat, torch.zeros(1, 64)).numpy()
    assert np.frombuffer(rec[0, 512:516].tobytes(), "<f4")[0] == 256.0


# ----------------------------------------------------------------- attention pins

@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_tiny(seed):
    q, kv, ip, ix = tiny_case(seed)
    out, lse = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    bo, bl = brute_force(q, kv, ip, ix, SIGMA)
    assert_close(out, bo, 1e-12)
    assert_close(lse, bl, 1e-12)


def test_dense_case_matches_sdpa():
    """Every row attends to every record: multi-query attention, one KV head."""
    rng = np.random.default_rng(7)
    T, H, N = 3, 5, 40
    kv = random_records(rng, N, scale_exp=(-8, 0))
    q = random_q(rng, T, H, std=2.0)
    ip = np.arange(T + 1) * N
    ix = np.tile(np.arange(N), T)
    out, lse = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    K = torch.from_numpy(torch_decode(kv))
    Q = torch.from_numpy(torch_q(q))
    qq = Q[:, :, None, :]
    kk = K[None, None].expand(T, H, N, 576)
    vv = K[None, None, :, :512].expand(T, H, N, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=SIGMA)[:, :, 0]
    scores = torch.matmul(Q, K.T) * SIGMA
    assert np.max(np.abs(out - ref.numpy())) <= 1e-10
    assert np.max(np.abs(lse - torch.logsumexp(scores, dim=-1).numpy())) <= 1e-10


def test_single_index_returns_row():
    rng = np.random.default_rng(3)
    kv = random_records(rng, 9)
    q = random_q(rng, 9, 4)
    ip = np.arange(10)
    ix = np.arange(9)[::-1].copy()
    out, lse = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    K = torch_decode(kv)
    Q = torch_q(q)
    for r in range(9):
        k = K[ix[r]]
        assert np.array_equal(out[r], np.broadcast_to(k[:512], (4, 512)))
        for h in range(4):
            want = SIGMA * math.fsum(float(a) * float(b) for a, b in zip(Q[r, h], k))
            assert abs(lse[r, h] - want) <= 1e-12 * max(1.0, abs(want))


def test_equal_scores_give_mean():
    rng = np.random.default_rng(4)
    kv = random_records(rng, 30)
    q = np.zeros((1, 2, 576), np.uint16)  # q = 0: every score is 0
    ix = rng.integers(0, 30, size=17)
    out, lse = oracle.sparse_mla_fwd(q, kv, [0, 17], ix, SIGMA)
    mean = torch_decode(kv[ix])[:, :512].mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) <= 1e-12 * max(1, np.abs(mean).max())
    assert np.allclose(lse, math.log(17), rtol=0, atol=1e-14)


def test_weighted_abs_value():
    """The oracle's A = p |V| / l: equal to out when every latent is >= 0, never
    below |out|, the plain mean of |V| when all scores are equal, and the same
    out and lse as without it."""
    rng = np.random.default_rng(14)
    kv = random_records(rng, 40)
    q = random_q(rng, 3, 4)
    ip = np.array([0, 25, 25, 40])
    ix = rng.integers(0, 40, size=40)
    o, l = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    o2, l2, A = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA, with_abs=True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    assert np.all(A >= np.abs(o) - 1e-12 * np.maximum(1.0, A))
    assert np.array_equal(A[1], np.zeros_like(A[1]))  # empty row
    pos = kv.copy()
    pos[:, :512] &= 0x7F  # clear every latent code's sign bit
    op, _, Ap = oracle.sparse_mla_fwd(q, pos, ip, ix, SIGMA, with_abs=True)
    assert np.max(np.abs(Ap - op)) <= 1e-12 * max(1.0, np.abs(op).max())
    q0 = np.zeros((1, 2, 576), np.uint16)  # equal scores: A is the mean of |V|
    _, _, A0 = oracle.sparse_mla_fwd(q0, kv, [0, 17], ix[:17], SIGMA, with_abs=True)
    want = np.abs(torch_decode(kv[ix[:17]])[:, :512]).mean(axis=0)
    assert np.max(np.abs(A0[0] - want)) <= 1e-12 * max(1.0, want.max())


def test_permutation_invariance():
    q, kv, ip, ix = tiny_case(100)
    rng = np.random.default_rng(5)
    ix2 = ix.copy()
    for r in range(len(ip) - 1):
        b, e = ip[r], ip[r + 1]
        ix2[b:e] = rng.permutation(ix[b:e])
    o1, l1 = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    o2, l2 = oracle.sparse_mla_fwd(q, kv, ip, ix2, SIGMA)
    assert_close(o2, o1, 1e-12)
    assert_close(l2, l1, 1e-12)


def test_negative_entries_ignored():
    rng = np.random.default_rng(6)
    kv = random_records(rng, 12)
    q = random_q(rng, 1, 3)
    base = np.array([3, 7, 0, 11, 5])
    withneg = np.array([-1, 3, -1, -1, 7, 0, -7, 11, 5, -1])
    o1, l1 = oracle.sparse_mla_fwd(q, kv, [0, 5], base, SIGMA)
    o2, l2 = oracle.sparse_mla_fwd(q, kv, [0, 10], withneg, SIGMA)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_duplicates_raise_lse_by_ln2():
    rng = np.random.default_rng(8)
    kv = random_records(rng, 12)
    q = random_q(rng, 1, 3)
    base = np.array([3, 7, 0, 11, 5])
    o1, l1 = oracle.sparse_mla_fwd(q, kv, [0, 5], base, SIGMA)
    o2, l2 = oracle.sparse_mla_fwd(q, kv, [0, 10], np.repeat(base, 2), SIGMA)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * max(1, np.abs(o1).max())
    assert np.max(np.abs(l2 - (l1 + math.log(2)))) <= 1e-12


def test_empty_rows():
    rng = np.random.default_rng(9)
    kv = random_records(rng, 4)
    q = random_q(rng, 4, 2)
    ip = np.array([0, 0, 3, 1, 4])  # row0 empty, row1 all -1, row2 negative length
    ix = np.array([-1, -1, -1, 2])
    out, lse = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    assert np.all(out[:3] == 0.0) and np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3]))


def test_index_out_of_range_raises():
    rng = np.random.default_rng(10)
    kv = random_records(rng, 4)
    with pytest.raises(IndexError):
        oracle.sparse_mla_fwd(random_q(rng, 1, 1), kv, [0, 2], [1, 4], SIGMA)


def test_lse_merge_equals_unsplit():
    rng = np.random.default_rng(11)
    kv = random_records(rng, 50, scale_exp=(-8, 2))
    q = random_q(rng, 1, 4, std=2.0)
    ix = rng.integers(-1, 50, size=37)
    whole = oracle.sparse_mla_fwd(q, kv, [0, 37], ix, SIGMA)
    for cuts in ([10, 20], [1, 2, 3, 36], [0, 0, 37], [5]):
        edges = [0] + list(cuts) + [37]
        parts = [oracle.sparse_mla_fwd(q, kv, [0, e - b], ix[b:e], SIGMA)
                 for b, e in zip(edges[:-1], edges[1:])]
        out, lse = oracle.lse_merge([(o[0], s[0]) for o, s in parts])
        assert np.max(np.abs(out - whole[0][0])) <= 1e-12 * max(1, np.abs(whole[0]).max())
        assert np.max(np.abs(lse - whole[1][0])) <= 1e-12


def test_lse_merge_all_empty():
    out, lse = oracle.lse_merge([(np.full((2, 512), np.nan), np.full(2, -np.inf))] * 3)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------- planted mistakes

def _pins_pass():
    """Run the attention pins; return the names of those that fail."""
    failed = []
    checks = [
        ("bruteforce", lambda: [test_bruteforce_tiny(s) for s in (0, 3, 5)]),
        ("sdpa", test_dense_case_matches_sdpa),
        ("single", test_single_index_returns_row),
        ("mean", test_equal_scores_give_mean),
        ("negative", test_negative_entries_ignored),
        ("dups", test_duplicates_raise_lse_by_ln2),
        ("empty", test_empty_rows),
        ("merge", test_lse_merge_equals_unsplit),
    ]
    for name, fn in checks:
        try:
            fn()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(name)
    return failed


def _mut_decode(fn):
    real = ocodec.decode_records

    def wrapped(rec):
        return fn(real(rec), rec)
    return wrapped


def _row_attention_variant(kind):
    def f(Q, K, sigma):
        H = Q.shape[0]
        if K.shape[0] == 0:
            return np.zeros((H, 512)), np.full(H, -np.inf)
        s = (Q @ K.T) * (1.0 if kind == "no_sigma" else sigma)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(m - s) if kind == "sign" else np.exp(s - m)
        l = p.sum(axis=1)
        V = K[::-1, :512] if kind == "transposed_v" else K[:, :512]
        out = (p @ V) / l[:, None]
        lse = m[:, 0] + (np.log2(l) if kind == "log2" else np.log(l))
        return out, lse
    return f


MUTANTS = {
    "rope_dropped": ("decode_records", _mut_decode(lambda K, rec: np.concatenate(
        [K[:, :512], np.zeros_like(K[:, 512:])], axis=1))),
    "scale_block_shift": ("decode_records", _mut_decode(lambda K, rec: np.concatenate(
        [K[:, :128], 2 * K[:, 128:256], K[:, 256:]], axis=1))),
    "no_sigma": ("row_attention", _row_attention_variant("no_sigma")),
    "sign": ("row_attention", _row_attention_variant("sign")),
    "log2_lse": ("row_attention", _row_attention_variant("log2")),
    "transposed_v": ("row_attention", _row_attention_variant("transposed_v")),
    "negatives_kept": ("_row_keys", lambda kv, sl: ocodec.decode_records(kv[sl])),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(monkeypatch, name):
    assert _pins_pass() == []
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oatt, attr, fn)
    failed = _pins_pass()
    assert failed, f"planted mistake {name!r} went unnoticed by every pin"


# ----------------------------------------------------------------- cache writer pins

import oracle.writer as owriter  # noqa: E402


def _e4m3_finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_e4m3_encode_roundtrips_every_code():
    """Every finite code's value encodes back to that code (-0.0 to 0x80)."""
    codes = np.array(_e4m3_finite_codes())
    vals = oracle.E4M3_TABLE[codes]
    assert np.array_equal(owriter.e4m3_encode(vals), codes.astype(np.uint8))


def test_e4m3_encode_ties_to_even():
    """The midpoint of two neighbouring codes goes to the one with the even
    mantissa; a hair above or below goes to the nearer one (closed form)."""
    for c in range(0, 0x7E):  # positive finite neighbours (c, c + 1)
        lo, hi = oracle.E4M3_TABLE[c], oracle.E4M3_TABLE[c + 1]
        mid = (lo + hi) / 2.0
        even = c if (c & 1) == 0 else c + 1
        assert owriter.e4m3_encode(mid) == even, hex(c)
        assert owriter.e4m3_encode(-mid) == (0x80 | even), hex(c)
        eps = (hi - lo) * 2.0 ** -20
        assert owriter.e4m3_encode(mid - eps) == c
        assert owriter.e4m3_encode(mid + eps) == c + 1


def test_e4m3_encode_matches_torch():
    """Library routine: torch's float8_e4m3fn cast (round to nearest even)."""
    rng = np.random.default_rng(21)
    y = np.concatenate([
        rng.uniform(-448.0, 448.0, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),           # subnormal range
        np.ldexp(rng.uniform(-1, 1, 20000), rng.integers(-12, 9, 20000)),
    ])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(owriter.e4m3_encode(y), ref)


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        owriter.e4m3_encode(np.array([449.0]))


def test_pow2ceil_closed_form(golden):
    for k in range(-30, 20):
        assert owriter.pow2ceil(2.0 ** k) == 2.0 ** k
        assert owriter.pow2ceil(2.0 ** k * (1 + 2.0 ** -40)) == 2.0 ** (k + 1)
        assert owriter.pow2ceil(2.0 ** k * 0.75) == 2.0 ** k
    for amax, scale in golden("writer_bound.txt"):
        assert owriter.pow2ceil(max(float(amax), owriter.AMAX_FLOOR) / 448.0) == float(scale)


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_writer_records_decode_within_half_step():
    """Decoding a written record gives each latent value back within half an
    e4m3 step of its magnitude times the block scale, and the rope exactly;
    every block's largest value lands in (224, 448] times the scale."""
    rng = np.random.default_rng(22)
    n = 64
    x = rng.standard_normal((n, 512)) * np.exp(rng.uniform(-12, 8, (n, 4))).repeat(128, axis=1)
    x[:4, :128] = 0.0  # floored blocks
    lb = _bf16_bits(x)
    rb = _bf16_bits(rng.standard_normal((n, 64)))
    rec = owriter.encode_records(lb, rb)
    K = oracle.decode_records(rec)
    xb = oracle.bf16_bits_to_f64(lb)
    sc = np.frombuffer(rec[:, 512:528].tobytes(), "<f4").reshape(n, 4).astype(np.float64)
    s = np.repeat(sc, 128, axis=1)
    y = np.abs(xb) / s
    step = np.where(y >= 2.0 ** -6, np.ldexp(1.0, np.frexp(np.maximum(y, 2.0 ** -6))[1] - 4), 2.0 ** -9)
    assert np.all(np.abs(K[:, :512] - xb) <= 0.5 * step * s)
    assert np.array_equal(K[:, 512:], oracle.bf16_bits_to_f64(rb))
    amax = np.abs(xb).reshape(n, 4, 128).max(axis=2)
    live = amax >= 1e-4
    assert np.all((amax / sc)[live] <= 448.0) and np.all((amax / sc)[live] > 224.0)
    assert np.all(sc[~live] == 2.0 ** -22)


def test_writer_matches_generator_rule():
    """The oracle writer and the workload generator (torch casts) store the
    same bytes for bf16 inputs."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((32, 512)) * 3.0
    x[:, 5] = 1000.0
    lb, rb = _bf16_bits(x), _bf16_bits(rng.standard_normal((32, 64)))
    lat = torch.from_numpy(oracle.bf16_bits_to_f64(lb).astype(np.float32))
    rope = torch.from_numpy(oracle.bf16_bits_to_f64(rb).astype(np.float32))
    assert np.array_equal(owriter.encode_records(lb, rb), synth.encode_records(lat, rope).numpy())


def test_write_cache_slots():
    rng = np.random.default_rng(24)
    kv = rng.integers(0, 256, size=(10, 656), dtype=np.uint8)
    lb, rb = _bf16_bits(rng.standard_normal((4, 512))), _bf16_bits(rng.standard_normal((4, 64)))
    out = owriter.write_cache(kv, lb, rb, [7, -1, 2, 10])
    rec = owriter.encode_records(lb, rb)
    assert np.array_equal(out[7], rec[0]) and np.array_equal(out[2], rec[2])
    untouched = [i for i in range(10) if i not in (2, 7)]
    assert np.array_equal(out[untouched], kv[untouched])


@pytest.mark.parametrize("name", ["half_away", "scale_floor", "no_floor"])
def test_writer_planted_mistakes(monkeypatch, name):
    """Plausible writer mistakes, planted in the oracle, fail some writer pin."""
    checks = [test_e4m3_encode_ties_to_even, test_e4m3_encode_matches_torch,
              test_writer_records_decode_within_half_step]
    if name == "half_away":
        monkeypatch.setattr(np, "rint", lambda v: np.floor(np.asarray(v) + 0.5))
    elif name == "scale_floor":
        def floor2(x):
            m, e = np.frexp(np.asarray(x, np.float64))
            return np.ldexp(1.0, (e - 1).astype(np.int64))
        monkeypatch.setattr(owriter, "pow2ceil", floor2)
    else:
        monkeypatch.setattr(owriter, "AMAX_FLOOR", 0.0)
    failed = 0
    for fn in checks:
        try:
            fn()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed += 1
    assert failed, f"planted writer mistake {name!r} went unnoticed"


# ----------------------------------------------------------------- paged pools and sink pins

import oracle.paged as opaged  # noqa: E402


def paged_case(seed):
    rng = np.random.default_rng(seed)
    N, T, H = 40, 5, 3
    kv = random_records(rng, N, scale_exp=(-6, 0))
    q = torch.from_numpy(rng.standard_normal((T, H, 576)).astype(np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lens = [7, 0, 12, 1, 20]
    ip = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ix = np.concatenate([rng.integers(0, N, L) for L in lens]).astype(np.int64)
    ix[3] = -1
    return rng, kv, q, ip, ix


@pytest.mark.parametrize("seed", range(4))
def test_paged_equals_contiguous(seed):
    """The same keys through two paged pools give exactly the contiguous result."""
    rng, kv, q, ip, ix = paged_case(seed)
    pools, entry_of = paged_layout(rng, kv)
    pix = np.where(ix >= 0, entry_of[np.maximum(ix, 0)], -1)
    assert np.any(pix < -1) and np.any(pix >= 0)  # both pools in use
    ro, rl = oracle.sparse_mla_fwd(q, kv, ip, ix, SIGMA)
    po, pl = opaged.sparse_mla_fwd_paged(q, pools, ip, pix, SIGMA)
    assert np.array_equal(ro, po) and np.array_equal(rl, pl)


def test_paged_entry_decoding():
    """-1 is no key; other negatives select the compressed pool by their low 31 bits."""
    pools = [(np.zeros(10 * 656, np.uint8), 5 * 656, 5), (np.zeros(4 * 1000, np.uint8), 1000, 1)]
    assert opaged.resolve(-1, pools) is None
    assert opaged.resolve(7, pools) == (0, 1 * 5 * 656 + 2 * 656)
    assert opaged.resolve(np.int32(np.uint32((1 << 31) | 3)), pools) == (1, 3 * 1000)
    with pytest.raises(IndexError):
        opaged.resolve(10, pools)


def test_sink_none_equals_minus_inf():
    rng, kv, q, ip, ix = paged_case(7)
    pools, entry_of = paged_layout(rng, kv)
    pix = np.where(ix >= 0, entry_of[np.maximum(ix, 0)], -1)
    a = opaged.sparse_mla_fwd_paged(q, pools, ip, pix, SIGMA)
    b = opaged.sparse_mla_fwd_paged(q, pools, ip, pix, SIGMA, sink=np.full(3, -np.inf))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sink_closed_form_equal_scores():
    """q = 0: every logit is 0, so out = mean(V) n / (n + e^sink) and lse = ln(n + e^sink)."""
    rng = np.random.default_rng(8)
    K = oracle.decode_records(random_records(rng, 9, scale_exp=(-6, 0)))
    sink = np.array([-3.0, 0.0, 2.5])
    out, lse = opaged.row_attention_sink(np.zeros((3, 576)), K, SIGMA, sink)
    n = K.shape[0]
    want = K[:, :512].mean(axis=0)[None, :] * (n / (n + np.exp(sink)))[:, None]
    assert np.allclose(out, want, rtol=0, atol=1e-13)
    assert np.allclose(lse, np.log(n + np.exp(sink)), rtol=0, atol=1e-13)


def test_sink_bruteforce_extra_key():
    """Pure-Python softmax over the n logits plus the sink logit, the sink's value 0."""
    rng = np.random.default_rng(9)
    K = oracle.decode_records(random_records(rng, 6, scale_exp=(-4, 0)))
    Q = rng.standard_normal((2, 576))
    sink = np.array([0.7, -1.2])
    out, lse = opaged.row_attention_sink(Q, K, SIGMA, sink)
    for h in range(2):
        logits = [SIGMA * float(np.dot(Q[h], K[j])) for j in range(6)] + [float(sink[h])]
        mx = max(logits)
        ws = [math.exp(x - mx) for x in logits]
        tot = sum(ws)
        for d in (0, 100, 511):
            v = sum(ws[j] * K[j, d] for j in range(6)) / tot
            assert abs(out[h, d] - v) <= 1e-12 * max(1.0, abs(v))
        assert abs(lse[h] - (mx + math.log(tot))) <= 1e-12


def test_sink_is_one_more_merged_part():
    """Chunk results without the sink, merged together with one extra part of
    out 0 and lse = sink (stage_combine's fold), equal the unsplit forward with
    the sink; this is how split rows take their sink."""
    rng, kv, q, ip, ix = paged_case(9)
    pools, entry_of = paged_layout(rng, kv)
    pix = np.where(ix >= 0, entry_of[np.maximum(ix, 0)], -1)
    sink = np.array([1.0, -np.inf, 6.0])
    whole = opaged.sparse_mla_fwd_paged(q, pools, ip, pix, SIGMA, sink=sink)
    for r in range(len(ip) - 1):
        b, e = int(ip[r]), int(ip[r + 1])
        for cuts in ([], [b + (e - b) // 2], [b, b + 1, e]):
            edges = [b] + [c for c in cuts if b <= c <= e] + [e]
            parts = []
            for lo, hi in zip(edges[:-1], edges[1:]):
                o, l = opaged.sparse_mla_fwd_paged(q[r:r + 1], pools, [0, hi - lo], pix[lo:hi], SIGMA)
                parts.append((o[0], l[0]))
            parts.append((np.zeros((3, 512)), sink))
            out, lse = oracle.lse_merge(parts)
            assert np.max(np.abs(out - whole[0][r])) <= 1e-12 * max(1.0, np.abs(whole[0][r]).max())
            fin = np.isfinite(whole[1][r])
            assert np.array_equal(np.isfinite(lse), fin)
            assert np.max(np.abs(lse[fin] - whole[1][r][fin]), initial=0.0) <= 1e-12


def test_sink_empty_row():
    out, lse = opaged.row_attention_sink(np.zeros((2, 576)), np.zeros((0, 576)), SIGMA, np.array([1.5, -np.inf]))
    assert np.all(out == 0.0) and lse[0] == 1.5 and lse[1] == -np.inf


@pytest.mark.parametrize("name", ["sink_in_numerator", "sink_not_exponentiated", "pool_bit_ignored"])
def test_paged_planted_mistakes(monkeypatch, name):
    real_row, real_resolve = opaged.row_attention_sink, opaged.resolve
    if name == "sink_in_numerator":
        def f(Q, K, sigma, sink):
            out, lse = real_row(Q, K, sigma, sink)
            if sink is None or K.shape[0] == 0:
                return out, lse
            s = sigma * (Q @ K.T)
            m = np.maximum(s.max(axis=1), sink)
            w = np.exp(np.asarray(sink) - m) / np.exp(lse - m)
            return out + w[:, None] * K[0, :512][None, :], lse
        monkeypatch.setattr(opaged, "row_attention_sink", f)
    elif name == "sink_not_exponentiated":
        def f(Q, K, sigma, sink):
            if sink is None or K.shape[0] == 0:
                return real_row(Q, K, sigma, sink)
            s = sigma * (Q @ K.T)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1) + np.asarray(sink)
            return (p @ K[:, :512]) / l[:, None], m + np.log(np.abs(l))
        monkeypatch.setattr(opaged, "row_attention_sink", f)
    else:
        monkeypatch.setattr(opaged, "resolve", lambda e, pools: None if int(e) == -1
                            else real_resolve(int(e) & 0x7FFFFFFF, pools))
    failed = 0
    for fn in (lambda: [test_paged_equals_contiguous(s) for s in range(2)], test_sink_closed_form_equal_scores,
               test_sink_bruteforce_extra_key):
        try:
            fn()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed += 1
    assert failed, f"planted mistake {name!r} went unnoticed"
