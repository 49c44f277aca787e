"""GPU parity of the cache writer (sparse_mla_cache_write, through the C ABI)
against the fp64 oracle writer: the written bytes must be identical.

Every case prints its name and shape before touching the GPU.  Inputs are
seeded and synthetic; the oracle never sees anything the HIP path produced.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from parity import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_fp8_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def varied_latent(rng, n):
    """N(0,1) latent with a per-block magnitude over 2^-30 .. 2^15, plus the
    edge cases: all-zero and floored blocks, -0.0, values in e4m3's subnormal
    range, +-1000 outliers and values that land exactly halfway between two
    e4m3 codes after scaling."""
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(-30, 15, (n, 4))).repeat(128, axis=1)
    x[0, :128] = 0.0
    x[1, :] = -0.0
    x[2, 128:256] = 3e-5                           # below the 1e-4 floor
    x[3, :] = rng.standard_normal(512) * 2.0 ** -12
    x[3, 0] = 448.0                                # scale 1: small values hit e4m3 subnormals
    x[4, rng.integers(0, 512, 20)] = rng.choice([-1000.0, 1000.0], 20)
    codes = np.array([c for c in range(0x7E)])     # positive finite codes below 448
    mids = (oracle.E4M3_TABLE[codes] + oracle.E4M3_TABLE[codes + 1]) / 2.0
    for r in range(5, min(n, 9)):                  # block 0 amax 448 -> scale 1; ties in the rest
        x[r, 0] = 448.0
        x[r, 1:128] = rng.choice(mids, 127) * rng.choice([-1.0, 1.0], 127)
    return x


def test_cache_write_bitexact(smla):
    rng = np.random.default_rng(40)
    n, N = 3000, 4096
    lat = bf16(varied_latent(rng, n))
    rope = bf16(rng.standard_normal((n, 64)))
    slots = rng.permutation(N)[:n].astype(np.int64)
    kv0 = rng.integers(0, 256, size=(N, 656), dtype=np.uint8)  # untouched rows keep these bytes
    note(f"cache_write n={n} N={N}")
    kv = torch.from_numpy(kv0).to(DEV)
    smla.cache_write(lat.to(DEV), rope.to(DEV), torch.from_numpy(slots).to(DEV), kv)
    torch.cuda.synchronize()
    got = kv.cpu().numpy()
    want = oracle.write_cache(kv0, bits(lat), bits(rope), slots)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first (row, byte): {bad[:5].tolist()}, " \
                          f"got {got[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}"


def test_cache_write_skips_padding_and_out_of_range(smla):
    rng = np.random.default_rng(41)
    n, N = 64, 50
    lat = bf16(rng.standard_normal((n, 512)))
    rope = bf16(rng.standard_normal((n, 64)))
    slots = np.full(n, -1, np.int64)
    slots[::3] = rng.permutation(N)[: len(slots[::3])]
    slots[1] = N          # out of range: skipped
    slots[2] = 1 << 40    # far out of range: skipped
    kv0 = rng.integers(0, 256, size=(N, 656), dtype=np.uint8)
    note(f"cache_write skips n={n} N={N}")
    kv = torch.from_numpy(kv0).to(DEV)
    smla.cache_write(lat.to(DEV), rope.to(DEV), torch.from_numpy(slots).to(DEV), kv)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), oracle.write_cache(kv0, bits(lat), bits(rope), slots))


def test_cache_write_strided_inputs(smla):
    rng = np.random.default_rng(42)
    n, N = 200, 300
    big = bf16(rng.standard_normal((n, 576)) * 5.0)   # latent and rope as views of one [n, 576] row
    slots = rng.permutation(N)[:n].astype(np.int64)
    kv0 = np.zeros((N, 656), np.uint8)
    note(f"cache_write strided n={n}")
    big_d = big.to(DEV)
    kv = torch.from_numpy(kv0).to(DEV)
    smla.cache_write(big_d[:, :512], big_d[:, 512:], torch.from_numpy(slots).to(DEV), kv)
    torch.cuda.synchronize()
    want = oracle.write_cache(kv0, bits(big[:, :512].contiguous()), bits(big[:, 512:].contiguous()), slots)
    assert np.array_equal(kv.cpu().numpy(), want)


def test_cache_write_large(smla):
    """A 65,536-record cache written in one call (the decode workload's size)."""
    rng = np.random.default_rng(43)
    N = 65536
    lat = bf16(rng.standard_normal((N, 512)))
    rope = bf16(rng.standard_normal((N, 64)))
    slots = rng.permutation(N).astype(np.int64)
    note(f"cache_write large N={N}")
    kv = torch.zeros(N, 656, dtype=torch.uint8, device=DEV)
    smla.cache_write(lat.to(DEV), rope.to(DEV), torch.from_numpy(slots).to(DEV), kv)
    torch.cuda.synchronize()
    want = oracle.write_cache(np.zeros((N, 656), np.uint8), bits(lat), bits(rope), slots)
    assert np.array_equal(kv.cpu().numpy(), want)


def test_quantize_then_attend(smla):
    """End to end: records written by the GPU writer, attended by the GPU
    forward, match the oracle's forward over the oracle writer's records."""
    import synth
    rng = np.random.default_rng(44)
    N, T, H, k = 3000, 6, 16, 700
    lat = bf16(rng.standard_normal((N, 512)) * 2.0)
    rope = bf16(rng.standard_normal((N, 64)))
    slots = np.arange(N, dtype=np.int64)
    sl = [rng.choice(N, k, replace=False) for _ in range(T)]
    w = synth.build_workload("writer_e2e", T, H, N, lambda g, r, m: sl[r], seed=45, device="cpu")
    w.kv = torch.from_numpy(oracle.write_cache(np.zeros((N, 656), np.uint8), bits(lat), bits(rope), slots))
    note(f"quantize then attend N={N} T={T}")
    kv = torch.zeros(N, 656, dtype=torch.uint8, device=DEV)
    smla.cache_write(lat.to(DEV), rope.to(DEV), torch.from_numpy(slots).to(DEV), kv)
    torch.cuda.synchronize()
    assert torch.equal(kv.cpu(), w.kv)
    wg = w.to(DEV)
    wg.kv = kv
    out, lse = run_gpu(wg)
    ro, rl = run_oracle(w)
    compare(out, lse, ro, rl, label="writer_e2e")
