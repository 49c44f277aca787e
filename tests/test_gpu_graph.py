"""Capture of the library's calls in a HIP graph.

Every call takes its outputs and workspace from the caller and neither
allocates, synchronises nor clears memory with a memset, so a sequence of
calls can be captured on a stream.  These tests capture a few calls, replay
the graph several times with eager calls and synchronisations in between, and
require every replay's outputs to equal the eager call's bit for bit.  The
outputs are overwritten with a fill value before each replay, so a replay
that wrote nothing would fail.

Cases: the decode shape (split + combine), a ragged batch with masked entries
and more units than compute units (plan scan and sort kernels), the paged
pools with a sink, and the V4.1 record with its MXFP8 epilogue.  A last test
runs two problems on two streams at once.
"""

import sys

import numpy as np
import pytest
import torch

import synth
import synth.v41 as sv
from pools import paged_layout, v41_layout

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_fp8_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.set_option("split", 0)
    m.set_option("plan", 0)
    return m


def replay_check(step, outputs, replays=4, calls=3):
    """Eager reference, capture of `calls` calls, then `replays` replays each
    checked against the reference.  `outputs` returns the output tensors (the
    ones the captured calls write)."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            step()
    torch.cuda.synchronize()
    for r in range(replays):
        for t in outputs():
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, rt) in enumerate(zip(outputs(), ref)):
            assert torch.equal(t, rt), f"replay {r}: output {i} differs from the eager call"
        step()  # eager work between the replays
        torch.cuda.synchronize()
    del g


def test_graph_decode(smla):
    T, H, N, k = 16, 16, 8192, 1024
    w = synth.build_workload("graph_decode", T, H, N, lambda g, r, m: np.sort(synth.distinct_uniform(g, N, k)),
                             seed=3, device="cuda")
    note(f"graph decode T={T} H={H} N={N} k={k} split={smla.split_for(T, H, w.nnz)}")
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = smla.workspace(DEV, smla.workspace_bytes(T, H, w.nnz))

    def step():
        smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, out=out, lse=lse, ws=ws)

    replay_check(step, lambda: [out, lse])


def test_graph_ragged_plan(smla):
    T, H, N = 300, 16, 16384
    rng = np.random.default_rng(4)
    lens = rng.integers(1, 513, T)

    def rows(g, r, m):
        s = synth.distinct_uniform(g, N, int(lens[r]))
        s = np.where(torch.rand(len(s), generator=g).numpy() < 0.05, -1, s)
        return np.concatenate([s, -np.ones(512 - len(s), np.int64)])

    w = synth.build_workload("graph_ragged", T, H, N, rows, seed=5, device="cuda", has_invalid=1)
    S = smla.split_for(T, H, w.nnz, True)
    note(f"graph ragged T={T} H={H} N={N} rows of 1..512 keys padded to 512, split={S}")
    assert T * S > 256, "the case should run the plan kernels"
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = smla.workspace(DEV, smla.workspace_bytes(T, H, w.nnz))

    def step():
        smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, has_invalid=True, out=out, lse=lse, ws=ws)

    replay_check(step, lambda: [out, lse])


def test_graph_paged_sink(smla):
    T, H, N, k = 24, 16, 8192, 700
    w = synth.build_workload("graph_paged", T, H, N, lambda g, r, m: synth.distinct_uniform(g, N, k),
                             seed=6, device="cpu")
    rng = np.random.default_rng(6)
    pools, entry_of = paged_layout(rng, w.kv.numpy())
    ix = w.indices.numpy().astype(np.int64)
    ent = torch.from_numpy(np.where(ix >= 0, entry_of[np.maximum(ix, 0)], -1).astype(np.int32)).to(DEV)
    pools_d = [(torch.from_numpy(np.ascontiguousarray(b)).to(DEV), st, pr) for b, st, pr in pools]
    sink = torch.from_numpy(rng.normal(0.0, 3.0, H).astype(np.float32)).to(DEV)
    q, indptr = w.q.to(DEV), w.indptr.to(DEV)
    note(f"graph paged+sink T={T} H={H} N={N} k={k}")
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = smla.workspace(DEV, smla.workspace_bytes(T, H, int(ent.numel())))

    def step():
        smla.fwd_paged(q, pools_d, indptr, ent, w.sm_scale, sink=sink, out=out, lse=lse, ws=ws)

    replay_check(step, lambda: [out, lse])


def test_graph_v41(smla):
    T, H, N, k = 16, 16, 4096, 600
    rng = np.random.default_rng(7)
    data, scales = sv.make_v41_keys(N, seed=7)
    pools, entry_of = v41_layout(rng, data, scales)
    ind = np.concatenate([entry_of[rng.permutation(N)[:k]] for _ in range(T)]).astype(np.int32)
    indices = torch.from_numpy(ind).to(DEV)
    indptr = torch.arange(0, T * k + 1, k, dtype=torch.int32, device=DEV)
    pools_d = [(torch.from_numpy(b).to(DEV), st, pr) for b, st, pr in pools]
    q = sv.make_q(T, H, seed=8).to(DEV)
    cos_sin = torch.from_numpy(sv.make_cos_sin(1024)).to(DEV)
    pos = torch.from_numpy(rng.integers(0, 1024, T).astype(np.int32)).to(DEV)
    sink = torch.from_numpy(rng.normal(0.0, 2.0, H).astype(np.float32)).to(DEV)
    ws = smla.workspace(DEV, smla.v41_workspace_bytes(T, H, T * k))
    note(f"graph v41 T={T} H={H} N={N} k={k}")
    held = {}

    def step():
        held["o"] = smla.fwd_v41(q, pools_d, indptr, indices, sv.sm_scale_v41(), pos, cos_sin, sink=sink, ws=ws)

    # the captured calls' outputs live in the graph's memory pool; the eager
    # calls between replays allocate their own, so compare what the capture
    # returned
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in held["o"]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    captured = held["o"]
    torch.cuda.synchronize()
    for r in range(4):
        for t in captured:
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, rt) in enumerate(zip(captured, ref)):
            assert torch.equal(t, rt), f"replay {r}: output {i} differs from the eager call"
        step()
        torch.cuda.synchronize()
    del g


def test_concurrent_streams(smla):
    """Two streams, each with its own workspace, run different problems with
    their calls interleaved and no synchronisation between them; each result
    equals that problem's result run alone, bit for bit (the library keeps no
    state shared between calls besides what the caller passes)."""
    N = 16384
    a = synth.build_workload("streams_a", 32, 16, N, lambda g, r, m: synth.distinct_uniform(g, N, 700),
                             seed=21, device="cuda")
    rng = np.random.default_rng(22)
    lens = rng.integers(1, 600, 280)

    def rows(g, r, m):
        s = synth.distinct_uniform(g, N, int(lens[r]))
        return np.concatenate([s, -np.ones(600 - len(s), np.int64)])

    b = synth.build_workload("streams_b", 280, 16, N, rows, seed=23, device="cuda", has_invalid=1)
    note("concurrent streams: decode 32 x 700 keys (split + combine) and ragged 280 rows (plan kernels)")
    outs = {}
    for name, w, hi in (("a", a, False), ("b", b, True)):
        o = torch.empty(w.T, w.H, 512, dtype=torch.bfloat16, device=DEV)
        l = torch.empty(w.T, w.H, dtype=torch.float32, device=DEV)
        ws = torch.empty(smla.workspace_bytes(w.T, w.H, w.nnz), dtype=torch.uint8, device=DEV)
        outs[name] = (w, hi, o, l, ws)
    ref = {}
    for name, (w, hi, o, l, ws) in outs.items():
        smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, has_invalid=hi, out=o, lse=l, ws=ws)
        torch.cuda.synchronize()
        ref[name] = (o.clone(), l.clone())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for name, _, _, o, l, _ in [(k, *v) for k, v in outs.items()]:
        o.fill_(7)
        l.fill_(7)
    torch.cuda.synchronize()
    for _ in range(6):
        for name, st in (("a", s1), ("b", s2)):
            w, hi, o, l, ws = outs[name]
            with torch.cuda.stream(st):
                smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, has_invalid=hi, out=o, lse=l, ws=ws)
    torch.cuda.synchronize()
    for name, (w, hi, o, l, ws) in outs.items():
        assert torch.equal(o, ref[name][0]) and torch.equal(l, ref[name][1]), f"problem {name} differs"


def test_two_graphs_default_workspace_replayed_at_once(smla):
    """Two graphs captured one after the other with the binding's default
    workspace (both captures run on torch's one default capture stream), then
    replayed at the same time on two streams: each capture got a workspace of
    its own from its graph's memory pool, so each replay equals its eager
    result bit for bit."""
    T, H, N, k = 32, 16, 16384, 1024
    ws_ = [synth.build_workload(f"graphs_{i}", T, H, N, lambda g, r, m: np.sort(synth.distinct_uniform(g, N, k)),
                                seed=31 + i, device="cuda") for i in range(2)]
    note(f"two graphs: {T} x {k} keys each, split {smla.split_for(T, H, T * k)}, replayed on two streams at once")
    outs = [(torch.empty(T, H, 512, dtype=torch.bfloat16, device=DEV),
             torch.empty(T, H, dtype=torch.float32, device=DEV)) for _ in ws_]
    ref = []
    for w, (o, l) in zip(ws_, outs):
        smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, out=o, lse=l)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
    graphs = []
    for w, (o, l) in zip(ws_, outs):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, out=o, lse=l)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(3):
                smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, out=o, lse=l)
        torch.cuda.synchronize()
        graphs.append(g)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for r in range(4):
        for o, l in outs:
            o.fill_(7)
            l.fill_(7)
        torch.cuda.synchronize()
        for g, st in zip(graphs, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                g.replay()
        torch.cuda.synchronize()
        for i, ((o, l), (ro, rl)) in enumerate(zip(outs, ref)):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"replay {r}: graph {i} differs from its eager call"
    del graphs
