"""sparse_mla_fwd_noalloc (the forward with the library's static per-device
scratch in place of a workspace) against sparse_mla_fwd, through the C ABI.

Two no-allocation calls in a row, the second with a smaller input, both
using split partials in the scratch.  Each must give exactly the bytes that
sparse_mla_fwd gives on the same inputs (the same kernels on the same
split), and the smaller case is also checked against the fp64 oracle.  Runs
alone in a fresh process and after the other tests alike: the scratch keeps
the last call's contents, and nothing in it needs to start at zero.
"""

import sys

import numpy as np
import pytest
import torch

import synth
from parity import compare, run_oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def small_ragged():
    """5 rows x 7 heads over 4,096 records: slices of 700, 1, 0, 333 and 129
    keys in a stride of 700 entries, padded with -1 (has_invalid)."""
    lens = [700, 1, 0, 333, 129]

    def rows(g, r, m):
        k = lens[r]
        ix = synth.distinct_uniform(g, 4096, k) if k else np.zeros(0, np.int64)
        return np.concatenate([ix, -np.ones(700 - k, np.int64)])
    return synth.build_workload("ragged_T5_H7_N4096", len(lens), 7, 4096, rows, seed=77,
                                has_invalid=1, device="cuda")


def c_abi_noalloc(b, w, out, lse):
    rc = b.lib().sparse_mla_fwd_noalloc(
        w.q.data_ptr(), w.q.stride(0), w.q.stride(1), w.kv.data_ptr(), w.kv.shape[0],
        w.indptr.data_ptr(), w.indices.data_ptr(), w.nnz, w.T, w.H, w.sm_scale, w.has_invalid,
        out.data_ptr(), out.stride(0), out.stride(1), lse.data_ptr(),
        torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == 0, b.lib().sparse_mla_last_error()


def c_abi_workspace(b, w, out, lse):
    nb = b.workspace_bytes(w.T, w.H, w.nnz)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    rc = b.lib().sparse_mla_fwd(
        w.q.data_ptr(), w.q.stride(0), w.q.stride(1), w.kv.data_ptr(), w.kv.shape[0],
        w.indptr.data_ptr(), w.indices.data_ptr(), w.nnz, w.T, w.H, w.sm_scale, w.has_invalid,
        out.data_ptr(), out.stride(0), out.stride(1), lse.data_ptr(), ws.data_ptr(), nb,
        torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == 0, b.lib().sparse_mla_last_error()
    torch.cuda.synchronize()


def test_noalloc_two_calls_match_workspace_forward():
    from sparse_mla_decode_fp8_amd import binding as b
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    b.set_option("split", 0)
    big = synth.make_workload(2, device="cuda")   # 64 rows x 2,048 sorted keys, 16 heads: split 4
    small = small_ragged()                         # 5 rows, 7 heads: split 6
    cases = [big, small]
    for w in cases:
        note(f"{w.name}: T={w.T} H={w.H} nnz={w.nnz} split={b.split_for(w.T, w.H, w.nnz, bool(w.has_invalid))}")
        assert b.split_for(w.T, w.H, w.nnz, bool(w.has_invalid)) > 1
        assert b.workspace_bytes(w.T, w.H, w.nnz) <= b.NOALLOC_SCRATCH_BYTES
    # the two no-allocation calls, back to back on one stream (poisoned outputs)
    got = []
    for w in cases:
        out = torch.full((w.T, w.H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((w.T, w.H), float("nan"), dtype=torch.float32, device=DEV)
        c_abi_noalloc(b, w, out, lse)
        got.append((out, lse))
    torch.cuda.synchronize()
    for w, (out, lse) in zip(cases, got):
        ref_o = torch.full_like(out, float("nan"))
        ref_l = torch.full_like(lse, float("nan"))
        c_abi_workspace(b, w, ref_o, ref_l)
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"{w.name}: out differs"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"{w.name}: lse differs"
        note(f"{w.name}: no-allocation call equals the workspace call bit for bit")
    # the smaller case against the oracle as well
    ro, rl = run_oracle(small)
    err = compare(got[1][0], got[1][1], ro, rl, label=small.name)
    note(f"{small.name}: vs oracle {err}")


def test_noalloc_rejects_scratch_overflow():
    from sparse_mla_decode_fp8_amd import binding as b
    b.set_option("split", 32)
    try:
        T, H, nnz = 100, 128, 100 * 4096   # forced 32 chunks: 100 x 32 x 128 heads of partials
        assert b.workspace_bytes(T, H, nnz) > b.NOALLOC_SCRATCH_BYTES
        q = torch.zeros(T, H, 576, dtype=torch.bfloat16, device=DEV)
        kv = torch.zeros(16, 656, dtype=torch.uint8, device=DEV)
        ip = torch.arange(0, nnz + 1, 4096, dtype=torch.int32, device=DEV)
        ix = torch.zeros(nnz, dtype=torch.int32, device=DEV)
        out = torch.zeros(T, H, 512, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(b.SmlaError) as e:
            b.fwd_noalloc(q, kv, ip, ix, 0.04, out)
        assert e.value.status == b.SMLA_EWORKSPACE
        torch.cuda.synchronize()
        assert not out.any()   # nothing was queued
    finally:
        b.set_option("split", 0)
