"""Pins of the V4.1 oracle (oracle/v41.py) against what the pages and the
mathematics fix: hand-built records with closed-form values, the page's
address formula on a worked example, brute force, special cases that reduce
to library routines (torch's bf16 and float8_e4m3fn casts), rotation
identities, and planted mistakes that must each fail a pin."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.v41 as ov
import synth.v41 as sv
from pools import compressed_entry, v41_layout

SIGMA = float(np.float32(1.0 / math.sqrt(512)))


def bf16_bits(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- record

def test_e8m0_values():
    assert ov.e8m0_value(127) == 1.0
    assert ov.e8m0_value(0) == 2.0 ** -127
    assert ov.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(ov.e8m0_value(255))
    assert ov.e8m0_value(120) == 2.0 ** -7


def test_decode_handbuilt_record():
    """Every nope code 0x40 (e4m3 2.0), scale byte c = 120 + c, so dims
    64c .. 64c+63 equal 2 * 2^(c - 7); rope 64 x bf16 1.5 (bits 0x3FC0) except
    rope dim 5 = -0.25 (0xBE80)."""
    data = np.zeros((1, 576), np.uint8)
    data[0, :448] = 0x40
    rope = np.full(64, 0x3FC0, np.uint16)
    rope[5] = 0xBE80
    data[0, 448:] = rope.astype("<u2").view(np.uint8)
    scales = np.zeros((1, 8), np.uint8)
    scales[0, :7] = 120 + np.arange(7)
    scales[0, 7] = 255                      # the unused byte is never read
    K = ov.decode_v41(data, scales)[0]
    for c in range(7):
        assert np.all(K[64 * c:64 * c + 64] == 2.0 * 2.0 ** (c - 7))
    want_rope = np.full(64, 1.5)
    want_rope[5] = -0.25
    assert np.array_equal(K[448:], want_rope)


def test_decode_generator_records_within_half_step():
    """The generator's keys decode to their source values within half an e4m3
    step at the block's scale (relative 2^-4), and amax / scale <= 448."""
    data, scales = sv.make_v41_keys(64, seed=3, sigma=3.0)
    K = ov.decode_v41(data, scales)
    sc = ov.e8m0_value(scales[:, :7])
    assert np.all(np.abs(K[:, :448]).reshape(64, 7, 64).max(axis=2) <= 448.0 * sc)
    assert np.all(np.isfinite(K))


def test_key_address_worked_example():
    """key_rec with 4 keys a page and a 2368-byte page stride: window slot 6 is
    page 1, offset 2 -> data at 2368 + 2 * 576 = 3520 and scales at
    2368 + 4 * 576 + 2 * 8 = 4688; compressed slot 1 (bit 31 set) of a pool
    with 2 keys a page -> data 576, scales 2 * 576 + 8 = 1160."""
    pools = [(np.zeros(4 * 2368, np.uint8), 2368, 4), (np.zeros(3 * 1168, np.uint8), 1168, 2)]
    assert ov.resolve_v41(-1, pools) is None
    assert ov.resolve_v41(6, pools) == (0, 3520, 4688)
    assert ov.resolve_v41(int(compressed_entry(1)), pools) == (1, 576, 1160)
    with pytest.raises(IndexError):
        ov.resolve_v41(16, pools)


def test_gather_through_pages_returns_the_keys():
    rng = np.random.default_rng(5)
    data, scales = sv.make_v41_keys(40, seed=5)
    pools, entry_of = v41_layout(rng, data, scales, per_page=(8, 4), pad=(48, 16))
    order = rng.permutation(40)
    d, s = ov.gather_v41(pools, list(entry_of[order]) + [-1])
    assert np.array_equal(d, data[order]) and np.array_equal(s, scales[order])


# ----------------------------------------------------------------- attention

def test_single_key_returns_the_key():
    """One key: out = K (all 512 dims, rope included: V = K), lse = sigma q.k."""
    rng = np.random.default_rng(6)
    data, scales = sv.make_v41_keys(1, seed=6)
    K = ov.decode_v41(data, scales)
    Q = rng.standard_normal((3, 512))
    out, lse = ov.attention_v41(Q, K, SIGMA, None)
    assert np.allclose(out, np.broadcast_to(K, (3, 512)), rtol=0, atol=1e-12)
    assert np.allclose(lse, SIGMA * (Q @ K[0]), rtol=0, atol=1e-12)


def test_equal_scores_mean_with_sink():
    """q = 0: every logit 0, so out = mean(K) n / (n + e^s), lse = ln(n + e^s)."""
    data, scales = sv.make_v41_keys(9, seed=7)
    K = ov.decode_v41(data, scales)
    sink = np.array([-np.inf, 0.0, 1.7])
    out, lse = ov.attention_v41(np.zeros((3, 512)), K, SIGMA, sink)
    n = 9
    want = K.mean(axis=0)[None, :] * (n / (n + np.exp(sink)))[:, None]
    assert np.allclose(out, want, rtol=0, atol=1e-12)
    assert np.allclose(lse, np.log(n + np.exp(sink)), rtol=0, atol=1e-13)


def test_bruteforce_tiny():
    """Pure-Python softmax over the logits plus the sink logit (value 0)."""
    rng = np.random.default_rng(8)
    data, scales = sv.make_v41_keys(5, seed=8, sigma=2.0)
    K = ov.decode_v41(data, scales)
    Q = rng.standard_normal((2, 512))
    sink = np.array([0.3, -2.0])
    out, lse = ov.attention_v41(Q, K, SIGMA, sink)
    for h in range(2):
        logits = [SIGMA * sum(float(Q[h, d]) * float(K[j, d]) for d in range(512)) for j in range(5)]
        m = max(logits + [float(sink[h])])
        w = [math.exp(x - m) for x in logits]
        L = sum(w) + math.exp(float(sink[h]) - m)
        for d in (0, 63, 64, 447, 448, 449, 511):
            assert abs(out[h, d] - sum(w[j] * K[j, d] for j in range(5)) / L) <= 1e-12
        assert abs(lse[h] - (m + math.log(L))) <= 1e-12


def test_fwd_paged_rows_and_empty():
    """The row-level forward over pages equals attention over the gathered keys;
    an empty row and an all -1 row give out 0 and lse = sink."""
    rng = np.random.default_rng(9)
    data, scales = sv.make_v41_keys(30, seed=9)
    pools, entry_of = v41_layout(rng, data, scales)
    q = sv.make_q(3, 2, seed=9).view(torch.int16).numpy().view(np.uint16)
    sl = [entry_of[rng.permutation(30)[:11]], np.array([], np.int64), np.array([-1, -1])]
    ip = np.concatenate([[0], np.cumsum([len(s) for s in sl])])
    ix = np.concatenate(sl)
    sink = np.array([0.5, -1.0])
    out, lse = ov.sparse_mla_fwd_v41(q, pools, ip, ix, SIGMA, sink=sink)
    d, s = ov.gather_v41(pools, sl[0])
    o0, l0 = ov.attention_v41(oracle.bf16_bits_to_f64(q[0]), ov.decode_v41(d, s), SIGMA, sink)
    assert np.array_equal(out[0], o0) and np.array_equal(lse[0], l0)
    for r in (1, 2):
        assert np.all(out[r] == 0) and np.array_equal(lse[r], sink)


# ----------------------------------------------------------------- epilogue

def test_bf16_round_matches_torch():
    """Round to nearest even bf16: torch's float32 -> bfloat16 cast agrees on
    f32-representable inputs (normals, subnormals, exact ties)."""
    rng = np.random.default_rng(10)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 100, 20000)),
        (np.arange(1, 2000) * 2.0 ** -7 + 2.0 ** -9) * np.exp2(rng.integers(-20, 20, 1999)),  # ties
        [0.0, -0.0, 2.0 ** -133, 3 * 2.0 ** -134, 1.0 + 2.0 ** -8],
    ]).astype(np.float32).astype(np.float64)
    want = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ov.bf16_round(x), want)


def test_inverse_rope_identities():
    rng = np.random.default_rng(11)
    o = rng.standard_normal((3, 512))
    ang = rng.uniform(-10, 10, 32)
    c, s = np.cos(ang), np.sin(ang)
    # cos 1, sin 0: identity; nope dims always untouched
    assert np.array_equal(ov.inverse_rope_gptj(o, np.ones(32), np.zeros(32)), o)
    y = ov.inverse_rope_gptj(o, c, s)
    assert np.array_equal(y[:, :448], o[:, :448])
    # cos 0, sin 1: e' = o, o' = -e
    y90 = ov.inverse_rope_gptj(o, np.zeros(32), np.ones(32))
    assert np.array_equal(y90[:, 448::2], o[:, 449::2]) and np.array_equal(y90[:, 449::2], -o[:, 448::2])
    # the GPT-J rotation by +angle (e cos - o sin, e sin + o cos) undone exactly
    fwd = o.copy()
    fwd[:, 448::2] = o[:, 448::2] * c - o[:, 449::2] * s
    fwd[:, 449::2] = o[:, 448::2] * s + o[:, 449::2] * c
    assert np.allclose(ov.inverse_rope_gptj(fwd, c, s), o, rtol=0, atol=1e-13)
    # pair norms preserved
    n0 = o[:, 448::2] ** 2 + o[:, 449::2] ** 2
    n1 = y[:, 448::2] ** 2 + y[:, 449::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)


def test_mx_exponent_rule():
    """E = floor(log2 amax) - 8, at least -127; 0 -> -127."""
    assert ov.mx_exponent(448.0) == 0
    assert ov.mx_exponent(256.0) == 0 and ov.mx_exponent(511.99) == 0 and ov.mx_exponent(512.0) == 1
    assert ov.mx_exponent(1.0) == -8 and ov.mx_exponent(1.999) == -8
    assert ov.mx_exponent(0.0) == -127 and ov.mx_exponent(1e-40) == -127
    assert ov.mx_exponent(2.0 ** 100) == 92


def test_mxfp8_round_trip_and_saturation():
    rng = np.random.default_rng(12)
    E = rng.integers(-40, 40, 50)
    codes = rng.integers(0, 0x7F, (50, 32)).astype(np.uint8)      # finite e4m3 magnitudes
    codes |= (rng.integers(0, 2, (50, 32)) << 7).astype(np.uint8)
    codes[:, 0] = 0x78 | (codes[:, 0] & 0x80)                       # |value| 256 = 2^8: fixes E
    y = oracle.E4M3_TABLE[codes] * np.exp2(E)[:, None]
    q, e8 = ov.mxfp8_quantize(y)
    assert np.array_equal(e8, (E + 127).astype(np.uint8)[:, None])
    assert np.array_equal(ov.mxfp8_dequantize(q, e8), y)            # exact round trip
    # scaled values in (448, 512) saturate to +-448
    z = np.zeros((1, 32))
    z[0, 0], z[0, 1], z[0, 2] = 500.0, -480.0, 3.0
    q2, e2 = ov.mxfp8_quantize(z)
    assert e2[0, 0] == 127
    assert np.array_equal(oracle.E4M3_TABLE[q2[0, :3]], [448.0, -448.0, 3.0])
    # an all-zero block: byte 0, codes 0
    q3, e3 = ov.mxfp8_quantize(np.zeros((1, 32)))
    assert e3[0, 0] == 0 and np.all(oracle.E4M3_TABLE[q3] == 0)


def test_mxfp8_ties_to_even_and_torch_cast():
    """Midpoints of neighbouring e4m3 values go to the even code; in general
    the codes equal torch's float8_e4m3fn cast of y / 2^E (after the clamp)."""
    codes = np.arange(0x40, 0x6F)
    mids = (oracle.E4M3_TABLE[codes] + oracle.E4M3_TABLE[codes + 1]) / 2
    y = np.zeros((1, 64))
    y[0, 0] = y[0, 32] = 256.0                  # both blocks: E = 0, so y / 2^E = y
    slots = np.array([i for i in range(64) if i % 32][: len(mids)])
    y[0, slots] = mids
    q, e8 = ov.mxfp8_quantize(y)
    assert np.all(e8 == 127)
    got = q[0, slots]
    assert np.all(got % 2 == 0) and np.all((got == codes) | (got == codes + 1))
    rng = np.random.default_rng(13)
    y = rng.standard_normal((200, 64)) * np.exp2(rng.uniform(-20, 20, (200, 1)))
    q, e8 = ov.mxfp8_quantize(y)
    E = e8.astype(np.int64) - 127
    scaled = np.clip(y.reshape(200, 2, 32) / np.exp2(E)[..., None], -448, 448).astype(np.float32)
    want = torch.tensor(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(200, 64)
    assert np.array_equal(q, want)


def test_epilogue_composition():
    """v41_epilogue = MXFP8(inverse_rope(bf16(out))) with the row's cos/sin."""
    rng = np.random.default_rng(14)
    out = rng.standard_normal((2, 3, 512)) * 5
    cs = sv.make_cos_sin(50)
    pos = np.array([7, 49])
    y, codes, e8 = ov.v41_epilogue(out, cs, pos)
    for t in range(2):
        c = cs[pos[t], :32].astype(np.float64)
        s = cs[pos[t], 32:].astype(np.float64)
        yt = ov.inverse_rope_gptj(ov.bf16_round(out[t]), c, s)
        assert np.array_equal(y[t], yt)
    assert np.array_equal((codes, e8)[0], ov.mxfp8_quantize(y)[0])
    # dequantised within half an e4m3 step of y (relative 2^-4 of the value, or
    # half the subnormal step 2^(E-9) near zero), except where the clamp to
    # 448 * 2^E saturates (values of the block's top binade above 448 * 2^E)
    dq = ov.mxfp8_dequantize(codes, e8)
    scale = np.repeat(np.exp2(e8.astype(np.int64) - 127), 32, axis=-1)
    step = np.maximum(np.abs(y) * 2.0 ** -4, scale * 2.0 ** -10)
    excess = np.maximum(np.abs(y) - 448.0 * scale, 0.0)
    assert np.all(np.abs(dq - y) <= step + excess)
    assert np.all(np.abs(dq) <= 448.0 * scale)


# ----------------------------------------------------------------- planted mistakes

def _v41_pins_pass():
    fails = []
    for name, f in [("decode", test_decode_handbuilt_record), ("address", test_key_address_worked_example),
                    ("single", test_single_key_returns_the_key), ("rope", test_inverse_rope_identities),
                    ("mxexp", test_mx_exponent_rule), ("mxrt", test_mxfp8_round_trip_and_saturation)]:
        try:
            f()
        except AssertionError:
            fails.append(name)
    return fails


@pytest.mark.parametrize("mutant", ["scale_byte_shift", "v_without_rope", "forward_rope",
                                    "mx_exponent_ceil", "scale_area_without_data"])
def test_v41_planted_mistakes(monkeypatch, mutant):
    assert _v41_pins_pass() == []
    if mutant == "scale_byte_shift":
        real = ov.decode_v41

        def f(data, scales):
            s2 = np.roll(np.asarray(scales), -1, axis=1)
            return real(data, s2)
        monkeypatch.setattr(ov, "decode_v41", f)
    elif mutant == "v_without_rope":
        real = ov.attention_v41

        def f(Q, K, sigma, sink):
            out, lse = real(Q, K, sigma, sink)
            out = out.copy()
            out[:, 448:] = 0.0
            return out, lse
        monkeypatch.setattr(ov, "attention_v41", f)
    elif mutant == "forward_rope":
        real = ov.inverse_rope_gptj

        def f(o, cos, sin):
            return real(o, cos, -np.asarray(sin))
        monkeypatch.setattr(ov, "inverse_rope_gptj", f)
    elif mutant == "mx_exponent_ceil":
        def f(amax):
            a = np.asarray(amax, np.float64)
            return np.where(a > 0, np.ceil(np.log2(np.where(a > 0, a, 1.0) / 448.0)), -127).astype(np.int64)
        monkeypatch.setattr(ov, "mx_exponent", f)
    elif mutant == "scale_area_without_data":
        real = ov.resolve_v41

        def f(entry, pools):
            r = real(entry, pools)
            if r is None:
                return r
            p, d, s = r
            per = pools[p][2]
            return p, d, s - per * 576
        monkeypatch.setattr(ov, "resolve_v41", f)
    assert _v41_pins_pass() != [], f"mutant {mutant} passed every pin"
