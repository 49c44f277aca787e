"""Benchmark of the sparse MLA forward (plan + forward + combine) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
    python bench.py --op cache_write [--records N]     # the record writer

One "step" is one call of the whole op on one batch of the workload.  Prints
one JSON line (the last line of stdout).  Inputs are seeded synthetic tensors
made on the device before timing.  The workload defaults to the decode batch
(64 query rows, 16 heads, 65,536 records, 2,048 keys per row).

Figures:
  value        gathered KV GB/s over the timed steps, warm (back-to-back calls);
               gathered bytes = 656 B x (CSR entries >= 0), counted once per entry
  rows_per_s   query rows per second, same timing
  cold         the same figures with a 1 GiB scratch write between calls (no
               cache reuse across calls); median of per-call HIP-event times
  roofline     the forward kernel alone: gathered bytes per launch / its mean
               launch time (HIP events the library records around each launch
               on the launch stream) against 8 TB/s HBM peak; `traffic` is the
               HBM bytes per launch from the committed rocprofv3 counter summary
               (null if that summary was taken from other kernel source)
  timing       how the timed loops were run.  Each loop is queued behind a GPU
               spin kernel long enough to cover the host's submission of the
               whole loop, so its launches run back to back on the GPU, as in
               a GPU-bound serving loop; `covered` says whether the spin did
               cover it.  This matters for the per-kernel times: an event pair
               per launch costs the host several times the launch itself, and
               without the spin the GPU idles between calls and each forward
               starts from an idle chip, whose XCDs begin the grid up to ~2 us
               apart.
  graph        (--graph-replays R, default 10, 0 skips it) the op captured into a
               HIP graph of 20 calls and replayed R times; every replay's outputs
               must equal the eager call's bit for bit (matches_eager).  A
               failure is reported here and does not stop the run.
  cpu_baseline the fp64 CPU oracle on the same workload on this host's cores
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gathered KV GB/s and query-rows/s (sparse MLA fwd, top-k 2048); % HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
RECORD_BYTES = 656
KERNEL_SRCS = [os.path.join(ROOT, "sparse_mla_decode_fp8_amd", "csrc", f)
               for f in ("smla_kernels.hip", "smla_wide.hip", "smla_wide64.hip", "smla_device.h", "smla_internal.h")]
COUNTERS = os.path.join(ROOT, "profiles", "fwd_decode_T64_H16_counters.txt")


def kernel_sha() -> str:
    """First 16 hex digits of the SHA-256 of the kernel sources, concatenated."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(config_name: str):
    """HBM bytes per forward launch from the committed counter summary, if it
    was measured on this workload with the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    with open(COUNTERS) as f:
        for line in f:
            m = re.match(r"^(\w+):\s*(\S+)", line.strip())
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256_16") != kernel_sha() or kv.get("workload") != config_name:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float, max_workers: int):
    """Time the fp64 oracle over the workload's rows: whole passes over all rows,
    repeated until budget_s, in a pool of spawned processes (fresh interpreters
    that never touch the GPU), one BLAS thread each."""
    import numpy as np
    import torch
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    q = w.q.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    args = (q, w.kv.cpu().numpy(), w.indptr.cpu().numpy(), w.indices.cpu().numpy(), w.sm_scale)
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0)), w.T))
    chunks = [list(range(i, w.T, workers)) for i in range(workers)]
    valid = w.valid_entries()
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                             initializer=_cb_init, initargs=args) as ex:
        list(ex.map(_cb_rows, [[0]] * workers))  # start-up and imports, untimed
        passes = 0
        t0 = time.perf_counter()
        while True:
            list(ex.map(_cb_rows, chunks))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s or passes >= 1000:
                break
    return {
        "value": round(RECORD_BYTES * valid * passes / dt / 1e9, 4),
        "unit": "GB/s",
        "rows_per_s": round(w.T * passes / dt, 2),
        "cores": workers,
        "kind": "oracle",
        "sample": f"{passes} full pass(es) over all {w.T} rows of the timed workload "
                  f"({dt:.1f} s wall, fp64 NumPy oracle, {workers} processes x 1 BLAS thread)",
        "cpu": _cpu_model(),
    }


_CB_ARGS = None


def _cb_init(*args):
    global _CB_ARGS
    _CB_ARGS = args
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _cb_rows(rows):
    import oracle
    q, kv, ip, ix, sc = _CB_ARGS
    oracle.sparse_mla_fwd(q, kv, ip, ix, sc, rows=rows)
    return len(rows)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class LoopTimer:
    """Runs timed loops with their launches queued behind a GPU spin (see
    `timing` in the module docstring)."""

    def __init__(self, torch, step):
        self.torch = torch
        self.step = step
        cuda = torch.cuda
        cuda._sleep(1000)
        a, b = cuda.Event(enable_timing=True), cuda.Event(enable_timing=True)
        a.record()
        cuda._sleep(2_000_000)
        b.record()
        cuda.synchronize()
        self.cycles_per_ms = 2_000_000 / max(a.elapsed_time(b), 1e-3)
        # host cost of one plain call (the queue is empty, so nothing blocks)
        n = 20
        cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        self.host_us = (time.perf_counter() - t0) / n * 1e6
        cuda.synchronize()
        self.covered = True

    def _spin(self, calls: int, factor: float):
        """Queues a spin covering `calls` launches at `factor` x the plain host
        cost each (+5 ms); returns the events around it and its planned ms."""
        cuda = self.torch.cuda
        ms = min(calls * self.host_us * factor / 1e3 + 5.0, 5000.0)
        s0, s1 = cuda.Event(enable_timing=True), cuda.Event(enable_timing=True)
        s0.record()
        cuda._sleep(int(self.cycles_per_ms * ms))
        s1.record()
        return s0, s1

    def _check(self, s0, s1, host_ms: float):
        self.covered = self.covered and host_ms <= s0.elapsed_time(s1)

    def op_ms(self, steps: int) -> float:
        """Mean device time per call over `steps` back-to-back calls."""
        cuda = self.torch.cuda
        cuda.synchronize()
        s0, s1 = self._spin(steps, 2.0)
        e0, e1 = cuda.Event(enable_timing=True), cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        host_ms = (time.perf_counter() - t0) * 1e3
        cuda.synchronize()
        self._check(s0, s1, host_ms)
        return e0.elapsed_time(e1) / steps

    def kernel_times(self, smla, steps: int):
        """The library's per-launch event times over `steps` calls (a
        KernelTimer with its .ms and .launches)."""
        cuda = self.torch.cuda
        cuda.synchronize()
        with smla.KernelTimer(steps) as kt:
            s0, s1 = self._spin(steps, 8.0)   # an event pair per launch costs the host more
            t0 = time.perf_counter()
            for _ in range(steps):
                self.step()
            host_ms = (time.perf_counter() - t0) * 1e3
        cuda.synchronize()
        self._check(s0, s1, host_ms)
        return kt

    def report(self) -> dict:
        return {"queued_behind_spin": True, "covered": self.covered,
                "host_us_per_call": round(self.host_us, 2)}


def graph_replays(torch, step, outputs, replays: int, calls: int = 20) -> dict:
    """The op captured `calls` times into one HIP graph and replayed; each
    replay's outputs must equal the eager call's.  Eager calls run between the
    replays.  Returns the mean device time per call over the replays."""
    cuda = torch.cuda
    step()
    cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = cuda.Stream()
    side.wait_stream(cuda.current_stream())
    with cuda.stream(side):
        for _ in range(3):
            step()
    cuda.current_stream().wait_stream(side)
    cuda.synchronize()
    g = cuda.CUDAGraph()
    with cuda.graph(g):
        for _ in range(calls):
            step()
    cuda.synchronize()
    total, ok = 0.0, True
    for _ in range(replays):
        for t in outputs:
            t.zero_()
        e0, e1 = cuda.Event(enable_timing=True), cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        cuda.synchronize()
        total += e0.elapsed_time(e1)
        ok = ok and all(torch.equal(t, r) for t, r in zip(outputs, ref))
        step()
        cuda.synchronize()
    del g
    return {"ms_per_step": round(total / (replays * calls), 5), "replays": replays,
            "calls_per_graph": calls, "matches_eager": ok}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=2,
                    help="workload number 1..5; 6: a 2,048-token causal prefill (row r attends to r + 1 keys)")
    ap.add_argument("--heads", type=int, default=None,
                    help="run the workload with this many heads instead of its own (e.g. 64 on the decode workload)")
    ap.add_argument("--cold-steps", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain device copies of known size (counter scaling)")
    ap.add_argument("--op", choices=("fwd", "fwd_paged", "fwd_v41", "cache_write"), default="fwd",
                    help="fwd: the sparse MLA forward (default); fwd_paged: the same workload "
                         "through two paged pools with a per-head sink; fwd_v41: V4.1 keys (448 e4m3 + "
                         "64 bf16 rope, E8M0 per 64) with the MXFP8 epilogue; cache_write: the record writer")
    ap.add_argument("--page-records", type=int, default=64, help="records per page (fwd_paged)")
    ap.add_argument("--records", type=int, default=65536, help="records written per call (cache_write)")
    ap.add_argument("--graph-replays", type=int, default=10,
                    help="also replay the op from a captured HIP graph this many times (fwd, fwd_paged; 0: skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import synth
    import sparse_mla_decode_fp8_amd as smla

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.op == "cache_write":
        return bench_cache_write(args, torch, smla, dev)
    if args.op == "fwd_v41":
        return bench_v41(args, torch, smla, dev)
    cfg = synth.make_config(args.config)
    if args.heads is not None:
        cfg["name"] = synth.heads_name(cfg["name"], args.heads)
    print(f"[bench] generating {cfg['name']}", file=sys.stderr, flush=True)
    w = synth.make_workload(args.config, device="cuda", H=args.heads)
    valid = w.valid_entries()
    gathered = RECORD_BYTES * valid
    flop = 2.0 * w.H * (576 + 512) * valid
    out = torch.empty(w.T, w.H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.T, w.H, dtype=torch.float32, device=dev)
    ws = smla.workspace(dev, smla.workspace_bytes(w.T, w.H, w.nnz))

    def step():
        smla.fwd(w.q, w.kv, w.indptr, w.indices, w.sm_scale, has_invalid=bool(w.has_invalid),
                 out=out, lse=lse, ws=ws)

    paged = None
    if args.op == "fwd_paged":
        pools, entries, sink = paged_inputs(torch, w, args.page_records, seed=args.config)
        paged = {"page_records": args.page_records, "pool_bytes": [int(b.numel()) for b, _, _ in pools],
                 "sink": "N(0, 3) per head"}

        def step():  # noqa: F811 (the paged variant of the same step)
            smla.fwd_paged(w.q, pools, w.indptr, entries, w.sm_scale, sink=sink,
                           has_invalid=bool(w.has_invalid), out=out, lse=lse, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lt = LoopTimer(torch, step)

    # ---- warm: K back-to-back steps
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ms_per_step = lt.op_ms(args.steps)

    # ---- per-kernel device time (events around each launch, on its stream)
    kt = lt.kernel_times(smla, args.steps)
    fwd_ms = kt.ms["fwd"] / max(kt.launches["fwd"], 1)

    # ---- cold: flush caches between calls
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.cold_steps):
        scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold_ms = statistics.median(cold)
    del scratch

    graph = None
    if args.graph_replays > 0:
        print(f"[bench] graph replays ({args.graph_replays})", file=sys.stderr, flush=True)
        try:
            graph = graph_replays(torch, step, [out, lse], args.graph_replays)
        except Exception as exc:  # reported, not fatal: the eager figures above stand
            torch.cuda.synchronize()
            graph = {"error": f"{type(exc).__name__}: {exc}"}

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    s = ms_per_step * 1e-3
    achieved = gathered / (fwd_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gathered / s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg["name"], "T": w.T, "H": w.H, "N": w.N, "topk": cfg["topk"],
            "nnz": w.nnz, "valid_entries": valid, "has_invalid": w.has_invalid,
            "record_bytes": RECORD_BYTES, "split": _split_of(smla, w),
        },
        "op": args.op,
        "rows_per_s": round(w.T / s, 1),
        "tflops": round(flop / s / 1e12, 2),
        "pct_hbm_peak": round(100.0 * gathered / s / 1e9 / HBM_PEAK_GBS, 2),
        "precision": "records e4m3 (exactly dequantised); QK bf16 MFMA, PV f16 MFMA, f32 accumulation and softmax",
        "cold": {
            "ms_per_call_median": round(cold_ms, 5),
            "value": round(gathered / (cold_ms * 1e-3) / 1e9, 2),
            "rows_per_s": round(w.T / (cold_ms * 1e-3), 1),
            "pct_hbm_peak": round(100.0 * gathered / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "calls": args.cold_steps,
        },
        "kernels_ms_per_call": {k: round(kt.ms[k] / max(kt.launches[k], 1), 5) if kt.launches[k] else 0.0
                                for k in kt.KINDS},
        "timing": lt.report(),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(cfg["name"]),
            "kernel": _fwd_kernel_name(w.H, w.T, _split_of(smla, w), kt.launches["plan"] > 0),
            "bytes_per_launch": gathered,
            "launch_ms": round(fwd_ms, 5),
        },
    }
    if graph is not None:
        result["graph"] = graph
    if paged is not None:
        result["metric"] = METRIC + ", paged two-pool keys + sink"
        result["config"]["workload"] = cfg["name"] + f"_paged{args.page_records}_sink"
        result["config"]["paged"] = paged
        result["roofline"]["traffic"] = read_traffic(result["config"]["workload"])
    if args.config in (5, 6):  # the causal prefills: the cache stays on chip, the MFMA bounds them
        tf = flop / (fwd_ms * 1e-3) / 1e12
        result["roofline"].update({"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                   "flop_per_launch": flop})
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, 16)
    print(json.dumps(result), flush=True)
    return 0


def paged_inputs(torch, w, per_page: int, seed: int):
    """The workload's records scattered over two paged pools (key_rec
    addressing: entries >= 0 window-pool slots, compressed-pool slots with bit
    31 set), each record in a random pool at a random slot, pages of
    per_page records with a 256-byte gap after each page; plus a per-head sink
    drawn from N(0, 3).  Returns (pools, entries int32 [nnz], sink f32 [H])."""
    dev = w.kv.device
    g = torch.Generator(device=dev)
    g.manual_seed(0xB00 + seed)
    N = w.kv.shape[0]
    pool_of = torch.randint(0, 2, (N,), generator=g, device=dev)
    entry_of = torch.empty(N, dtype=torch.int64, device=dev)
    pools = []
    for p in range(2):
        ids = torch.nonzero(pool_of == p).squeeze(1)
        n = int(ids.numel())
        stride = per_page * RECORD_BYTES + 256
        npages = max((n + per_page - 1) // per_page, 1)
        buf = torch.randint(0, 256, (npages * stride,), generator=g, device=dev, dtype=torch.uint8)
        if n:
            slots = torch.randperm(n, generator=g, device=dev)
            recs = buf.as_strided((npages, per_page, RECORD_BYTES), (stride, RECORD_BYTES, 1))
            recs[slots // per_page, slots % per_page] = w.kv[ids]
            entry_of[ids] = slots if p == 0 else slots - (1 << 31)   # bit 31 set, as int32
        pools.append((buf, stride, per_page))
    ix = w.indices.to(torch.int64)
    entries = torch.where(ix >= 0, entry_of[ix.clamp(min=0)], -1).to(torch.int32)
    sink = (torch.randn(w.H, generator=g, device=dev) * 3.0).float()
    return pools, entries, sink


V41_KEY_BYTES = 576 + 8   # data + scale word per key


def bench_v41(args, torch, smla, dev) -> int:
    """The V4.1 key record at the decode shape of one rank: 64 rows x 16 heads,
    2,048 distinct sorted keys per row out of 65,536, keys spread over a window
    and a compressed pool of 64-key pages, a per-head sink, MXFP8 output.
    Algorithmic bytes per gathered key: 576 data + 8 scale = 584."""
    import numpy as np
    import synth
    import synth.v41 as sv
    T, H, N, k, R = 64, 16, 65536, 2048, 64
    print("[bench] generating v41 decode workload", file=sys.stderr, flush=True)
    data, scales = sv.make_v41_keys(N, seed=41)
    gen = torch.Generator()
    gen.manual_seed(41)
    rows = [np.sort(synth.distinct_uniform(gen, N, k)) for _ in range(T)]
    rng = np.random.default_rng(41)
    pool_of = rng.integers(0, 2, N)
    entry_of = np.zeros(N, np.int64)
    pools = []
    for p in range(2):
        ids = np.flatnonzero(pool_of == p)
        slots = rng.permutation(len(ids)).astype(np.int64)
        stride = R * V41_KEY_BYTES
        npages = max((len(ids) + R - 1) // R, 1)
        buf = np.zeros(npages * stride, np.uint8)
        page, off = slots // R, slots % R
        buf[(page * stride + off * 576)[:, None] + np.arange(576)[None, :]] = data[ids]
        buf[(page * stride + R * 576 + off * 8)[:, None] + np.arange(8)[None, :]] = scales[ids]
        entry_of[ids] = slots if p == 0 else slots - (1 << 31)
        pools.append((torch.from_numpy(buf).to(dev), stride, R))
    indices = torch.from_numpy(np.concatenate([entry_of[r] for r in rows]).astype(np.int32)).to(dev)
    indptr = torch.arange(0, T * k + 1, k, dtype=torch.int32, device=dev)
    q = sv.make_q(T, H, seed=42).to(dev)
    cos_sin = torch.from_numpy(sv.make_cos_sin(4096)).to(dev)
    pos = torch.from_numpy(rng.integers(0, 4096, T).astype(np.int32)).to(dev)
    sink = (torch.randn(H, generator=gen) * 2.0).float().to(dev)
    ws = smla.workspace(dev, smla.v41_workspace_bytes(T, H, T * k))
    gathered = V41_KEY_BYTES * T * k

    def step():
        smla.fwd_v41(q, pools, indptr, indices, sv.sm_scale_v41(), pos, cos_sin, sink=sink, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lt = LoopTimer(torch, step)
    ms_per_step = lt.op_ms(args.steps)
    kt = lt.kernel_times(smla, args.steps)
    fwd_ms = kt.ms["fwd"] / max(kt.launches["fwd"], 1)
    achieved = gathered / (fwd_ms * 1e-3) / 1e9
    result = {
        "metric": "gathered KV GB/s (V4.1 key record, MXFP8 epilogue)",
        "value": round(gathered / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"v41_decode_T{T}_H{H}_N{N}_top{k}_page{R}", "T": T, "H": H, "N": N,
                   "topk": k, "page_records": R, "key_bytes": V41_KEY_BYTES,
                   "split": smla.split_for(T, H, T * k)},
        "op": "fwd_v41",
        "rows_per_s": round(T / (ms_per_step * 1e-3), 1),
        "kernels_ms_per_call": {kk: round(kt.ms[kk] / max(kt.launches[kk], 1), 5) if kt.launches[kk] else 0.0
                                for kk in kt.KINDS},
        "timing": lt.report(),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "smla_fwd41_kernel",
            "bytes_per_launch": gathered,
            "launch_ms": round(fwd_ms, 5),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


WRITE_READ_BYTES = 512 * 2 + 64 * 2 + 8   # bf16 latent + bf16 rope + int64 slot per token
WRITE_WRITTEN_BYTES = 656                  # one record per token


def bench_cache_write(args, torch, smla, dev) -> int:
    """The record writer on n tokens written to a permutation of n slots:
    algorithmic bytes per token = 1,160 read + 656 written."""
    n = args.records
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    lat = torch.randn(n, 512, generator=g, device=dev).to(torch.bfloat16)
    rope = torch.randn(n, 64, generator=g, device=dev).to(torch.bfloat16)
    slots = torch.randperm(n, generator=g, device=dev).to(torch.int64)
    kv = torch.empty(n, 656, dtype=torch.uint8, device=dev)
    per_call = n * (WRITE_READ_BYTES + WRITE_WRITTEN_BYTES)

    def step():
        smla.cache_write(lat, rope, slots, kv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lt = LoopTimer(torch, step)
    ms_per_step = lt.op_ms(args.steps)
    kt = lt.kernel_times(smla, args.steps)
    kms = kt.ms["cache_write"] / max(kt.launches["cache_write"], 1)
    achieved = per_call / (kms * 1e-3) / 1e9
    result = {
        "metric": "cache write GB/s (fp8_ds_mla records from bf16 latent + rope)",
        "value": round(per_call / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"cache_write_N{n}", "records": n,
                   "bytes_per_token": WRITE_READ_BYTES + WRITE_WRITTEN_BYTES},
        "records_per_s": round(n / (ms_per_step * 1e-3), 1),
        "timing": lt.report(),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "smla_cache_write_kernel",
            "bytes_per_launch": per_call,
            "launch_ms": round(kms, 5),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def _fwd_kernel_name(H: int, T: int, S: int, planned: bool) -> str:
    """The forward kernel the library launches for H heads (contiguous cache).
    With the plan and more blocks than whole XCDs of compute units, the 16-head
    (up to two blocks per CU) and wide-head kernels run their persistent-grid
    instances."""
    if 16 < H <= 32:
        return "smla_fwdw_kernel<2>"
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * ((T + 7) // 8) * S * ((H + 63) // 64)
    grid = (cus // 8) * 8
    # (the 16-head kernel takes the persistent grid only up to two units per CU)
    persistent = "true" if planned and blocks > grid and (H > 16 or blocks <= 2 * grid) else "false"
    if H <= 16:
        return f"smla_fwd16_kernel<{persistent}>"
    return f"smla_fwdw64_kernel<false, {persistent}>"


def _split_of(smla, w) -> int:
    from sparse_mla_decode_fp8_amd import binding
    return binding.split_for(w.T, w.H, w.nnz, bool(w.has_invalid))


if __name__ == "__main__":
    sys.exit(main())
