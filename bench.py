#!/usr/bin/env python3
"""Benchmark of the fused all-reduce epilogue + residual + RMSNorm (+ FP4) on
one MI355X.

A step is one fused call (all of: rank-ordered sum of N bf16 partials,
residual add, residual_out store, RMSNorm, bf16 store) over one batch of
synthetic input resident in HBM. The timed workload is the prefill bandwidth
shape: N = 8 partials, t = 4096 tokens, d = 8192 (64 MiB per partial), with
0.1% outlier rows in the residual. Buffer sets rotate so that no call can be
served from the 256 MB Infinity Cache.

`value` is GB/s counted as ((N + 2) reads + 2 writes) x t x d x 2 bytes, the
counting the workload definition asks for. `roofline.achieved` uses the
algorithmic bytes instead (N partials + residual + gamma read, residual_out +
y written).

The last stdout line is one compact JSON record. Besides the prefill figures
it carries `decode`: µs per call (p50 of graph replays) of every decode shape
(single token; the Llama-3-8B and Llama-3.1-70B decode steps as 64- and
160-call hipGraph chains, plain and LL-packed; the FP4 shapes at t <= 64)
against the measured floor of an empty kernel with the same launch in a graph
of the same length, and `prefill_t512`: the single-round prefill calls next to
a copy of the same byte mix in the same launch shape. Every secondary
measurement (`--all-extras`) goes to a JSON file, not to stdout.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--all-extras]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published peak
INFINITY_CACHE_BYTES = 256 << 20
METRIC = "fused kernel HBM GB/s (% of peak) at prefill; µs/call p50 at decode shapes"
_CSRC = os.path.join(ROOT, "reduce_residual_rmsnorm_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("arfuse_device.hpp", "arfuse_rows.hip",
                                                    "arfuse.hip")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ byte accounting

def plane_bytes(t: int, d: int) -> int:
    """One bf16 [t][d] tensor: t x d x 2 bytes (the all-reduce message size of
    tensor parallelism, independent of the rank count)."""
    return t * d * 2


def algorithmic_bytes(n: int, t: int, d: int, ll: bool = False, out: bool = True,
                      fp4: bool = False, residual: bool = True, norm: bool = True,
                      rout: bool = True, fp8: bool = False, reset: bool = False):
    """(read, write) bytes one fused call must move: N partials (twice the
    bytes when LL-packed), the residual and gamma (fp32) read; residual_out,
    and y (bf16) and/or FP4 codes + scales and/or FP8 codes written, plus the
    N slot planes refilled with the sentinel when the call resets a set.
    Without gamma (all-reduce only) nothing past residual_out is read or
    written."""
    P = plane_bytes(t, d)
    reads = n * P * (2 if ll else 1) + (P if residual else 0) + (4 * d if norm else 0)
    writes = (P if rout else 0) + (n * P if reset else 0)
    if norm:
        writes += (P if out else 0) + ((t * d // 2 + t * d // 16) if fp4 else 0)
        writes += t * d if fp8 else 0
    return reads, writes


def counted_bytes(n: int, t: int, d: int) -> int:
    """The workload's own counting: (N + 2) reads and 2 writes of t x d x 2."""
    return (n + 2 + 2) * plane_bytes(t, d)


def page_fused_bytes_per_token(d: int):
    """Per-token traffic of the fused kernel as the TensorRT-LLM deep dive
    (§6.4) accounts it: residual read, new residual and norm output written;
    the peer slots it reads are not counted there."""
    return 2 * d, 2 * 2 * d


def page_unfused_bytes_per_token(d: int):
    """Per-token traffic of the unfused path of the same table: the all-reduce
    kernel reads and writes the tensor, then residual+norm reads two tensors
    and writes two."""
    return 3 * 2 * d, 3 * 2 * d


def source_digest() -> str:
    """Hash of every device source the row kernel is built from."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ device helpers

def _dev():
    import torch
    return torch.device("cuda:0")


def dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev()).view(torch.bfloat16)


def dev_bytes(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


class PrefillSets:
    """`nsets` device copies of one call's inputs plus outputs, rotated so
    consecutive calls touch disjoint memory. The keyword arguments select a
    fusion pattern (see `algorithmic_bytes`); `reset` runs the sentinel
    layout and refills a separate slot set of N planes on every call."""

    def __init__(self, ci, nsets: int, fp4: bool = False, out: bool = True,
                 residual: bool = True, norm: bool = True, rout: bool = True,
                 fp8: bool = False, reset: bool = False):
        import torch
        self.ci = ci
        self.sets = []
        self.reset = reset
        self.plain = residual and norm and rout and not fp8 and not reset
        parts0 = [dev_bf16(p) for p in ci.partials]
        res0 = dev_bf16(ci.residual)
        gamma = torch.from_numpy(ci.gamma).to(_dev()) if norm else None
        t, d = ci.t, ci.d
        for s in range(nsets):
            parts = parts0 if s == 0 else [p.clone() for p in parts0]
            res = (res0 if s == 0 else res0.clone()) if residual else None
            o = torch.empty_like(res0) if (out and norm) else None
            ro = torch.empty_like(res0) if rout else None
            codes = torch.empty((t, d // 2), dtype=torch.uint8, device=_dev()) if fp4 else None
            scales = torch.empty((t, d // 16), dtype=torch.uint8, device=_dev()) if fp4 else None
            f8 = torch.empty((t, d), dtype=torch.uint8, device=_dev()) if fp8 else None
            slots = [torch.empty_like(res0) for _ in parts] if reset else None
            self.sets.append((parts, res, gamma, o, ro, codes, scales, f8, slots))
        # the sentinel layout can wait, so its calls take a status word
        self.status = torch.zeros(4, dtype=torch.int32, device=_dev()) if reset else None

    def call(self, i: int):
        import reduce_residual_rmsnorm_amd as arf
        parts, res, gamma, o, ro, codes, scales, f8, slots = self.sets[i % len(self.sets)]
        if self.plain:
            arf.arfuse_rmsnorm(parts, res, gamma, float(self.ci.eps), o, ro, codes, scales)
            return
        arf.arfuse_rmsnorm_ex(parts, res, gamma, float(self.ci.eps), o, ro, codes, scales,
                              t=self.ci.t, d=self.ci.d,
                              layout=arf.ARFUSE_LAYOUT_SENTINEL if self.reset else 0,
                              reset=slots, fp8_out=f8, fp8_inv_scale=4.0, status=self.status)


def n_sets_for(call_bytes: int) -> int:
    """Enough rotating sets that the bytes touched between two uses of a set
    exceed twice the Infinity Cache."""
    return max(2, math.ceil(2 * INFINITY_CACHE_BYTES / max(1, call_bytes)) + 1)


def time_calls(fn, steps: int, warmup: int):
    """Warm up, then time exactly `steps` calls between two events on the
    current stream, synchronized on both sides. Returns ms per call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(warmup + i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


# graph replays per decode measurement (bench.py --decode-reps: fewer under a
# profiler, which serializes and inflates every dispatch)
DECODE_REPS = 200


def set_decode_reps(reps: int) -> None:
    global DECODE_REPS
    DECODE_REPS = max(5, int(reps))


def time_graph(g, reps: int):
    """p10/p50/p90 (µs) of `reps` replays of a captured graph, each bracketed
    by its own events."""
    import torch
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, e in ev:
        s.record()
        g.replay()
        e.record()
    torch.cuda.synchronize()
    us = sorted(s.elapsed_time(e) * 1e3 for s, e in ev)
    q = lambda p: us[min(len(us) - 1, int(p * len(us)))]
    return dict(p10=q(0.1), p50=statistics.median(us), p90=q(0.9))


# ------------------------------------------------------------ decode chains

def decode_chain(n: int, t: int, d: int, k: int, ll: bool = False, fp4: bool = False,
                 out: bool = True, reps: int = 0, seed: int = 0, fp8: bool = False,
                 sentinel: bool = False, fresh=None, split: int = 0, norm: bool = True,
                 block_threads: int = 0, vpt: int = 0):
    """µs per call of a k-call chain captured in one graph (call c reads call
    c-1's residual_out), and of the same-length graph of the empty kernel
    with the same launch (the per-node floor). `sentinel` reads the slots in
    the sentinel layout and refills a second slot set on every call (the
    triple-buffer reset), `fp8` adds the FP8 output. `fresh` (default: LL
    only) gives every call its own partial buffers, as a peer's push would,
    instead of re-reading one set that stays in the caches. `split` > 1
    divides every row among that many workgroups (sums of squares exchanged
    through a workspace). `norm=False` is the all-reduce alone (no
    gamma: residual_out is the only output). `block_threads` and `vpt`
    override the launch shape (0: the library's choice)."""
    import numpy as np
    import torch

    import reduce_residual_rmsnorm_amd as arf
    import seeded_inputs as si

    ci = si.make_call(n, t, d, seed=seed, outlier_frac=0.001 if fp4 else 0.0)
    fresh = ll if fresh is None else fresh
    # per call: its own flag (LL, fresh) or one flag for the reused set
    flags = [ci.ll_base + (c if fresh else 0) for c in range(k)]
    nsets = k if fresh else 1
    if ll:
        packed = np.stack([si.ll_pack_all(ci.partials, flags[c]) for c in range(nsets)])
        pdev = dev_bytes(packed)
    else:
        pdev = dev_bf16(np.stack([ci.partials] * nsets))
    parts = [[pdev[c % nsets, i] for i in range(n)] for c in range(k)]
    res0 = dev_bf16(ci.residual)
    bufs = [torch.empty_like(res0), torch.empty_like(res0)]
    gamma = torch.from_numpy(ci.gamma).to(_dev()) if norm else None
    out = out and norm
    o = torch.empty_like(res0) if out else None
    codes = torch.empty((t, d // 2), dtype=torch.uint8, device=_dev()) if fp4 else None
    scales = torch.empty((t, d // 16), dtype=torch.uint8, device=_dev()) if fp4 else None
    status = torch.zeros(4, dtype=torch.int32, device=_dev())
    f8 = torch.empty((t, d), dtype=torch.uint8, device=_dev()) if fp8 else None
    slots = [torch.empty_like(res0) for _ in range(n)] if sentinel else None
    epi = ((arf.ARFUSE_EPI_BF16 if out else 0) | (arf.ARFUSE_EPI_FP4 if fp4 else 0)
           | (arf.ARFUSE_EPI_FP8 if fp8 else 0))
    lay = (arf.ARFUSE_LAYOUT_LL if ll else
           arf.ARFUSE_LAYOUT_SENTINEL if sentinel else arf.ARFUSE_LAYOUT_PLAIN)
    # the split that runs (ARFUSE_SPLIT_AUTO: the library's choice for the shape)
    launch = dict(block_threads=block_threads, vpt=vpt)
    info = arf.arfuse_query_launch(n, t, d, epi, layout=lay, split=split, **launch)
    eff = int(info.split)
    ws = (torch.zeros(int(info.workspace_bytes), dtype=torch.uint8, device=_dev())
          if info.workspace_bytes else None)
    sx = dict(split=split, workspace=ws, **launch)

    def enqueue():
        for c in range(k):
            rin = res0 if c == 0 else bufs[c % 2]
            rout = bufs[(c + 1) % 2]
            if ll:
                arf.arfuse_rmsnorm_ex(parts[c], rin, gamma, float(ci.eps), o, rout, codes, scales,
                                      layout=arf.ARFUSE_LAYOUT_LL, ll_flag=flags[c], max_polls=4,
                                      status=status, **sx)
            elif sentinel or fp8 or split != 0 or not norm or block_threads or vpt:
                arf.arfuse_rmsnorm_ex(parts[c], rin, gamma, float(ci.eps), o, rout, codes, scales,
                                      t=t, d=d, layout=arf.ARFUSE_LAYOUT_SENTINEL if sentinel else 0,
                                      max_polls=4, status=status, reset=slots, fp8_out=f8,
                                      fp8_inv_scale=4.0, **sx)
            else:
                arf.arfuse_rmsnorm(parts[c], rin, gamma, float(ci.eps), o, rout, codes, scales)

    def enqueue_floor():
        for _ in range(k):
            arf.arfuse_launch_floor(n, t, d, epi, layout=lay, split=split, **launch)

    enqueue()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf):
        enqueue_floor()
    reps = reps or DECODE_REPS
    chain = time_graph(g, reps)
    floor = time_graph(gf, reps)
    st = status.cpu().numpy().view(np.uint32)
    if st[0] != 0:
        raise RuntimeError("arrival reported bad during the benchmark: %s" % st)
    r = dict(n=n, t=t, d=d, calls=k, layout="ll" if ll else "sentinel" if sentinel else "plain",
             split=eff, split_requested="auto" if split == arf.ARFUSE_SPLIT_AUTO else max(1, split),
             norm=norm,
             fp4=fp4, fp8=fp8, reset=sentinel, fresh_partials=bool(fresh),
             grid=int(info.grid), block=int(info.block),
             us_per_call_p50=chain["p50"] / k, chain_us_p50=chain["p50"],
             chain_us_p10=chain["p10"], chain_us_p90=chain["p90"],
             floor_us_per_node_p50=floor["p50"] / k, floor_chain_us_p50=floor["p50"])
    r["ratio_to_floor"] = r["us_per_call_p50"] / r["floor_us_per_node_p50"]
    del g, gf
    return r


def prefill_gbps(n: int, t: int, d: int, steps: int, warmup: int, fp4=False, out=True, seed=0,
                 windows: int = 5, **pattern):
    """Throughput of one fused call shape with rotating buffer sets: the
    median of `windows` timed windows of `steps` calls each (a single window
    can catch a slow spell of the device). `pattern` takes the keyword
    arguments of `algorithmic_bytes` beyond the shape."""
    import seeded_inputs as si
    ci = si.make_call(n, t, d, seed=seed, outlier_frac=0.001)
    rd, wr = algorithmic_bytes(n, t, d, out=out, fp4=fp4, **pattern)
    sets = PrefillSets(ci, n_sets_for(rd + wr), fp4=fp4, out=out, **pattern)
    per_window = [time_calls(sets.call, steps, warmup if w == 0 else 0) for w in range(windows)]
    ms = statistics.median(per_window)
    r = dict(n=n, t=t, d=d, fp4=fp4, out=out, nsets=len(sets.sets), us_per_call=ms * 1e3,
             us_per_call_windows=[round(w * 1e3, 2) for w in per_window],
             read_bytes=rd, write_bytes=wr, algorithmic_gbps=(rd + wr) / (ms * 1e-3) / 1e9,
             **pattern)
    if not fp4 and not pattern:
        r["counted_gbps"] = counted_bytes(n, t, d) / (ms * 1e-3) / 1e9
    del sets
    return r


def mix_gbps(n_in: int, n_out: int, t: int, d: int, steps: int, warmup: int, windows: int = 5):
    """The byte mix of a fused call (n_in planes read, n_out written, bf16
    [t][d]) without its arithmetic, in the fused call's launch shape
    (arfuse_stream_mix), with rotating sets like prefill_gbps: the bandwidth
    ceiling of that call shape."""
    import torch

    import reduce_residual_rmsnorm_amd as arf
    P = plane_bytes(t, d)
    nsets = n_sets_for((n_in + n_out) * P)
    sets = [([torch.full((P,), 1, dtype=torch.uint8, device=_dev()) for _ in range(n_in)],
             [torch.empty(P, dtype=torch.uint8, device=_dev()) for _ in range(n_out)])
            for _ in range(nsets)]

    def call(i):
        ins, outs = sets[i % nsets]
        arf.arfuse_stream_mix(ins, outs, t, d)

    per_window = [time_calls(call, steps, warmup if w == 0 else 0) for w in range(windows)]
    ms = statistics.median(per_window)
    del sets
    return dict(n_in=n_in, n_out=n_out, t=t, d=d, nsets=nsets, us_per_call=ms * 1e3,
                bytes=(n_in + n_out) * P, gbps=(n_in + n_out) * P / (ms * 1e-3) / 1e9)


def time_calls_each(fn, steps: int, first: int = 0):
    """Per-call durations (ms) of `steps` back-to-back calls, from events
    recorded between them on the launch stream."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn(first + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def stream_copy_gbps(nbytes: int = 1 << 30, steps: int = 20):
    import torch

    import reduce_residual_rmsnorm_amd as arf
    a = torch.empty(nbytes, dtype=torch.uint8, device=_dev())
    b = torch.empty(nbytes, dtype=torch.uint8, device=_dev())
    a.fill_(1)
    ms = time_calls(lambda i: arf.arfuse_stream_copy(b if i % 2 == 0 else a,
                                                     a if i % 2 == 0 else b, nbytes),
                    steps, 3)
    return dict(bytes=nbytes, us=ms * 1e3, gbps=2 * nbytes / (ms * 1e-3) / 1e9)


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(ci, budget_s: float = 12.0):
    """The oracle (scalar C, one host thread) on full calls of the timed
    workload, repeated until about `budget_s` seconds; median time."""
    import oracle
    orc = oracle.default()
    times = []
    t_end = time.time() + budget_s
    while time.time() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    med = statistics.median(times)
    return dict(value=counted_bytes(ci.n, ci.t, ci.d) / med / 1e9, unit="GB/s", cores=1,
                kind="oracle",
                sample="%d full calls of n=%d t=%d d=%d on one host thread (median %.3f s/call; "
                       "host %s)" % (len(times), ci.n, ci.t, ci.d, med, _cpu_model()))


def cpu_baseline_threads(ci, threads: int, budget_s: float = 8.0):
    """The same oracle on the same calls, its rows cut into `threads` slices
    that run on parallel host threads (the C oracle runs without Python's
    lock). The oracle's arithmetic is untouched: this only measures what the
    host's cores give together."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    orc = oracle.default()
    bounds = [(ci.t * k // threads, ci.t * (k + 1) // threads) for k in range(threads)]

    def rows(b):
        a, e = b
        return orc.allreduce_rmsnorm(ci.partials[:, a:e], ci.residual[a:e], ci.gamma, ci.eps)

    times = []
    with ThreadPoolExecutor(threads) as ex:
        t_end = time.time() + budget_s
        while time.time() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            list(ex.map(rows, bounds))
            times.append(time.perf_counter() - t0)
            if len(times) >= 50:
                break
    med = statistics.median(times)
    return dict(value=counted_bytes(ci.n, ci.t, ci.d) / med / 1e9, unit="GB/s", cores=threads,
                kind="oracle",
                sample="%d full calls of n=%d t=%d d=%d, rows split over %d host threads "
                       "(median %.3f s/call; host %s)" % (len(times), ci.n, ci.t, ci.d, threads,
                                                          med, _cpu_model()))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------ traffic

def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, "row_kernel_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------ profile summaries

# One decode chain per row-kernel instance, so the trace's per-kernel rows
# are one chain each.
DECODE_PROFILED = ("decode_n8_t8_d8192_chain160", "decode_n8_t8_d8192_chain160_ll",
                   "decode_n8_t8_d8192_chain160_sentinel", "fp4_n4_t1_d8192_x100")
# the same instances with split rows (a run of their own: split is a launch
# argument, not an instance)
DECODE_SPLIT_PROFILED = ("decode_n8_t8_d8192_chain160_split4", "decode_n8_t8_d8192_chain160_ll_split4",
                         "decode_n8_t8_d8192_chain160_sentinel_split4", "fp4_n4_t1_d8192_x100_split8")

# single-round prefill calls (512 rows: one workgroup per row, two per CU),
# and the C4 call's byte mix without its arithmetic in the same launch shape
SMALL_PREFILL_PROFILED = ("prefill_n8_t512_d8192", "fp4_n4_t512_d8192", "mix_9r2w_t512_d8192")

# decode chains whose byte and latency counters are taken, one row-kernel
# instance each: LL (fresh words per call) with whole and split rows at N = 8
# and 4, and the plain N = 8 chain with whole and split rows
DECODE_COUNTED = ("decode_n8_t8_d8192_chain160_ll", "decode_n8_t8_d8192_chain160_ll_split8",
                  "decode_n4_t8_d8192_chain160_ll", "decode_n4_t8_d8192_chain160_ll_split8",
                  "decode_n8_t8_d8192_chain160", "decode_n8_t8_d8192_chain160_split8")

PROFILE_COMMANDS = {
    "trace": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
             "-d $OUT/prof_trace -o prefill -- python3 $REPO/bench.py --steps 50 "
             "--warmup 5 --no-extras --no-cpu-baseline",
    "pmc_prefill": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {C} --kernel-include-regex "
                   "row_kernel -f csv -d $OUT/pmc_prefill_{C} -o pmc -- python3 "
                   "$REPO/bench.py --steps 5 --warmup 1 --no-extras --no-cpu-baseline",
    "pmc_copy": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {C} --kernel-include-regex "
                "copy_kernel -f csv -d $OUT/pmc_copy_{C} -o pmc -- python3 "
                "$REPO/bench.py --copy-only",
    "trace_small": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
                   "-d $OUT/prof_small -o small -- python3 $REPO/bench.py "
                   + " ".join("--only-extra " + x for x in SMALL_PREFILL_PROFILED),
    "pmc_small": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {C} --kernel-include-regex "
                 "'row_kernel|mix_kernel' -f csv -d $OUT/pmc_small_{C} -o pmc -- python3 $REPO/bench.py "
                 + " ".join("--only-extra " + x for x in SMALL_PREFILL_PROFILED),
    "trace_decode": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
                    "-d $OUT/prof_decode -o decode -- python3 $REPO/bench.py --decode-reps 20 "
                    + " ".join("--only-extra " + x for x in DECODE_PROFILED),
    "trace_decode_split": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
                          "-d $OUT/prof_decode_split -o decode -- python3 $REPO/bench.py "
                          "--decode-reps 20 "
                          + " ".join("--only-extra " + x for x in DECODE_SPLIT_PROFILED),
    "trace_counted": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
                     "-d $OUT/prof_counted -o decode -- python3 $REPO/bench.py --decode-reps 10 "
                     + " ".join("--only-extra " + x for x in DECODE_COUNTED),
    "pmc_counted": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {C} --kernel-include-regex "
                   "'row_kernel|floor_kernel' -f csv -d $OUT/pmc_counted_{N} -o pmc -- python3 "
                   "$REPO/bench.py --decode-reps 10 "
                   + " ".join("--only-extra " + x for x in DECODE_COUNTED),
}
# the counter sets of the decode chains (one rocprofv3 run each): bytes fetched
# and written past the L2, and the L2's outstanding read requests to the
# fabric summed over cycles, whose ratio to the request count is the average
# time a read spends past the L2 (Little's law)
DECODE_COUNTER_SETS = {"fetch": "FETCH_SIZE", "write": "WRITE_SIZE",
                       "lat": "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum"}


def _bench_line(log_path):
    if not os.path.exists(log_path):
        return None
    with open(log_path) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line)
    return None


def _counter(path, kname):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if kname in r["Kernel_Name"]]
    return statistics.median(vals), len(vals)


def summarize_profiles(outdir: str, dest: str = PROFILES) -> None:
    """Write profiles/row_kernel_<workload>_{stats.md,traffic.json} (into
    `dest`) from the rocprofv3 outputs of PROFILE_COMMANDS under `outdir`
    (their $OUT)."""
    import csv
    global PROFILES
    PROFILES = dest
    name = "prefill_n8_t4096_d8192"
    os.makedirs(PROFILES, exist_ok=True)
    line = _bench_line(os.path.join(outdir, "prof_trace.log"))
    rows = list(csv.DictReader(open(os.path.join(outdir, "prof_trace", "prefill_kernel_stats.csv"))))
    md = ["# row_kernel, %s: rocprofv3 kernel statistics" % name, "",
          "Command (`$REPO` is the repository root, `$OUT` the output directory):", "",
          "    " + PROFILE_COMMANDS["trace"], "",
          "Kernel source sha256[:16]: `%s`" % (line or {}).get("kernel_source", "?"), "",
          "| kernel | calls | average µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        md.append("| `%s` | %s | %.2f | %.2f | %.2f | %s |" % (
            r["Name"].replace("(anonymous namespace)::", ""), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
    if line:
        rd, wr = algorithmic_bytes(8, 4096, 8192)
        md += ["", "The same run's bench line (HIP events over the %d timed calls): %.2f µs per call, "
               "%.1f GB/s counted, roofline.achieved %.1f GB/s algorithmic (%.1f%% of 8 TB/s)." % (
                   line["steps"], line["ms_per_step"] * 1e3, line["value"],
                   line["roofline"]["achieved"], 100 * line["roofline"]["frac"])]
    with open(os.path.join(PROFILES, "row_kernel_%s_stats.md" % name), "w") as f:
        f.write("\n".join(md) + "\n")

    copy_bytes = 1 << 30
    fetch, nf = _counter(os.path.join(outdir, "pmc_prefill_FETCH_SIZE", "pmc_counter_collection.csv"), "row_kernel")
    write, nw = _counter(os.path.join(outdir, "pmc_prefill_WRITE_SIZE", "pmc_counter_collection.csv"), "row_kernel")
    cfetch, _ = _counter(os.path.join(outdir, "pmc_copy_FETCH_SIZE", "pmc_counter_collection.csv"), "copy_kernel")
    cwrite, _ = _counter(os.path.join(outdir, "pmc_copy_WRITE_SIZE", "pmc_counter_collection.csv"), "copy_kernel")
    kf = copy_bytes / (cfetch * 1024)
    kw = copy_bytes / (cwrite * 1024)
    rd, wr = algorithmic_bytes(8, 4096, 8192)
    pline = _bench_line(os.path.join(outdir, "pmc_prefill_FETCH_SIZE.log")) or {}
    rec = {
        "workload": name,
        "source_sha256_16": pline.get("kernel_source"),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write, "dispatches": [nf, nw],
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": cfetch, "write_kib": cwrite,
                             "fetch_factor": kf, "write_factor": kw},
        "read_bytes_per_launch": fetch * 1024 * kf, "write_bytes_per_launch": write * 1024 * kw,
        "traffic_bytes_per_launch": round(fetch * 1024 * kf + write * 1024 * kw),
        "algorithmic_read_bytes": rd, "algorithmic_write_bytes": wr,
        "traffic_over_algorithmic": (fetch * 1024 * kf + write * 1024 * kw) / (rd + wr),
        "commands": [PROFILE_COMMANDS["pmc_prefill"].format(C=c) for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                    [PROFILE_COMMANDS["pmc_copy"].format(C=c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
    }
    with open(os.path.join(PROFILES, "row_kernel_%s_traffic.json" % name), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))
    for which in ("decode", "decode_split"):
        if os.path.exists(os.path.join(outdir, "prof_" + which, "decode_kernel_stats.csv")):
            summarize_decode_profile(outdir, which)
    if os.path.exists(os.path.join(outdir, "prof_small", "small_kernel_stats.csv")):
        summarize_small_prefill_profile(outdir, kf, kw)
    if os.path.exists(os.path.join(outdir, "prof_counted", "decode_kernel_stats.csv")):
        summarize_decode_counters(outdir, kf, kw)


# the row-kernel instances of SMALL_PREFILL_PROFILED, as the tracer names them
SMALL_PREFILL_KERNELS = {
    "prefill_n8_t512_d8192": ("row_kernel<8, 1, false, false, 1, 0>", dict(n=8, t=512, d=8192)),
    "fp4_n4_t512_d8192": ("row_kernel<4, 1, false, false, 2, 0>",
                          dict(n=4, t=512, d=8192, out=False, fp4=True)),
    "mix_9r2w_t512_d8192": ("mix_kernel<1, false>", dict(n=8, t=512, d=8192, mix=(9, 2))),
}


def summarize_small_prefill_profile(outdir: str, kf: float, kw: float) -> None:
    """profiles/row_kernel_prefill_t512_stats.md and _traffic.json: kernel
    durations and HBM bytes of the single-round prefill calls, the byte
    counters scaled by the copy calibration factors (kf, kw) of the same
    profile run."""
    import csv
    line = _bench_line(os.path.join(outdir, "prof_small.log")) or {}
    rows = list(csv.DictReader(open(os.path.join(outdir, "prof_small", "small_kernel_stats.csv"))))
    md = ["# row_kernel, single-round prefill calls (t = 512): rocprofv3 kernel statistics", "",
          "Command (`$REPO` is the repository root, `$OUT` the output directory):", "",
          "    " + PROFILE_COMMANDS["trace_small"], "",
          "Kernel source sha256[:16]: `%s`" % source_digest(), "",
          "Each call reads its own rotated buffer set (7 sets of 92 MB for N = 8; the "
          "FP4 call's sets likewise exceed the Infinity Cache). Under the tracer the "
          "dispatches run apart, so each kernel below ran alone on the device.", "",
          "| kernel | calls | average µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        md.append("| `%s` | %s | %.2f | %.2f | %.2f | %s |" % (
            r["Name"].replace("(anonymous namespace)::", ""), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
    rec = {"source_sha256_16": source_digest(), "copy_factors": {"fetch": kf, "write": kw},
           "commands": [PROFILE_COMMANDS["pmc_small"].format(C=c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "workloads": {}}
    md += ["", "HBM bytes per dispatch (`FETCH_SIZE`, `WRITE_SIZE`, median over the "
           "dispatches, scaled by the copy calibration of the same profile run):", "",
           "| workload | kernel µs (trace average) | read bytes | write bytes | "
           "over algorithmic | algorithmic GB/s at the trace average |", "|---|---|---|---|---|---|"]
    for label, (kname, shape) in SMALL_PREFILL_KERNELS.items():
        fetch, nf = _counter(os.path.join(outdir, "pmc_small_FETCH_SIZE", "pmc_counter_collection.csv"), kname)
        write, nw = _counter(os.path.join(outdir, "pmc_small_WRITE_SIZE", "pmc_counter_collection.csv"), kname)
        kw_shape = {k: v for k, v in shape.items() if k not in ("n", "t", "d", "mix")}
        if "mix" in shape:      # n_in planes read, n_out written
            rd, wr = (shape["mix"][0] * plane_bytes(shape["t"], shape["d"]),
                      shape["mix"][1] * plane_bytes(shape["t"], shape["d"]))
        else:
            rd, wr = algorithmic_bytes(shape["n"], shape["t"], shape["d"], **kw_shape)
        rb, wb = fetch * 1024 * kf, write * 1024 * kw
        avg = [float(r["AverageNs"]) / 1e3 for r in rows if kname in r["Name"]]
        rec["workloads"][label] = {"kernel": kname, "dispatches": [nf, nw], "read_bytes": rb,
                                   "write_bytes": wb, "algorithmic_read_bytes": rd,
                                   "algorithmic_write_bytes": wr,
                                   "traffic_over_algorithmic": (rb + wb) / (rd + wr),
                                   "trace_average_us": avg[0] if avg else None}
        md.append("| %s | %s | %.0f | %.0f | %.4f | %s |" % (
            label, "%.2f" % avg[0] if avg else "?", rb, wb, (rb + wb) / (rd + wr),
            "%.0f" % ((rd + wr) / (avg[0] * 1e-6) / 1e9) if avg else "?"))
    ex = line.get("extras", {})
    if ex:
        md += ["", "The same run's events (median window of back-to-back calls, tracer attached):", ""]
        for k, v in ex.items():
            md.append("- %s: %.2f µs per call" % (k, v["us_per_call"]))
    md += ["", "`mix_kernel` is `arfuse_stream_mix` with 9 planes read and 2 written per row: "
           "the C4 call's bytes in the C4 call's launch (512 workgroups of 1024 threads, "
           "the same non-temporal loads and stores), without the arithmetic. Its time is the "
           "ceiling of that launch shape."]
    with open(os.path.join(PROFILES, "row_kernel_prefill_t512_stats.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(PROFILES, "row_kernel_prefill_t512_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def summarize_decode_profile(outdir: str, which: str = "decode") -> None:
    """profiles/row_kernel_decode_chains_stats.md (or, for the split-row
    chains, row_kernel_decode_split_chains_stats.md): kernel durations of the
    decode chains next to the graph's time per node."""
    import csv
    line = _bench_line(os.path.join(outdir, "prof_%s.log" % which)) or {}
    rows = list(csv.DictReader(open(os.path.join(outdir, "prof_" + which, "decode_kernel_stats.csv"))))
    title = "decode chains" if which == "decode" else "decode chains with split rows"
    md = ["# row_kernel, %s: rocprofv3 kernel statistics" % title, "",
          "Command (`$REPO` is the repository root, `$OUT` the output directory):", "",
          "    " + PROFILE_COMMANDS["trace_" + which], "",
          "Kernel source sha256[:16]: `%s`" % line.get("kernel_source", "?"), "",
          "Each chain is captured once in a graph and replayed (5 warm-up + 200 timed "
          "replays), then the same-length graph of the empty kernel is replayed. Every "
          "row-kernel instance below belongs to exactly one chain.", "",
          "| kernel | calls | average µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        md.append("| `%s` | %s | %.2f | %.2f | %.2f | %s |" % (
            r["Name"].replace("(anonymous namespace)::", ""), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
    ex = line.get("extras", {})
    fl = [r for r in rows if "floor_kernel" in r["Name"]]
    if fl:
        md += ["", "The tracer adds time to every dispatch: the empty kernel itself averages "
               "%.2f µs here and a graph node of it takes the per-node time below, against "
               "1.6-1.7 µs untraced. Compare the instances with each other and with the empty "
               "kernel; bench.py's untraced extras give the per-call times." % (
                   float(fl[0]["AverageNs"]) / 1e3)]
    if ex:
        md += ["", "The same run's graph timings under the tracer (HIP events around each replay):", "",
               "| chain | µs per call (p50) | empty-kernel µs per node | ratio |", "|---|---|---|---|"]
        for k, v in ex.items():
            md.append("| %s | %.2f | %.2f | %.2f |" % (k, v["us_per_call_p50"],
                                                     v["floor_us_per_node_p50"], v["ratio_to_floor"]))
    fname = "row_kernel_decode_chains_stats.md" if which == "decode" else \
        "row_kernel_decode_split_chains_stats.md"
    with open(os.path.join(PROFILES, fname), "w") as f:
        f.write("\n".join(md) + "\n")


# the row-kernel instance of each counted decode chain, as the tracer names it
def _counted_shape(label):
    n = int(label.split("_n")[1].split("_")[0])
    return dict(n=n, t=8, d=8192, ll="_ll" in label,
                split=8 if "split8" in label else 1)


def _counted_kernel(label):
    sh = _counted_shape(label)
    return "row_kernel<%d, 1, %s, false, 1, %d>" % (sh["n"], "true" if sh["ll"] else "false",
                                                    1 if sh["split"] > 1 else 0)


def summarize_decode_counters(outdir: str, kf: float, kw: float) -> None:
    """profiles/row_kernel_decode_counters.md: per decode chain, the kernel's
    traced duration, bytes fetched and written past the L2 (scaled by the
    copy calibration), and the average time a fabric read request spends
    outstanding (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, in L2 clock cycles)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(outdir, "prof_counted", "decode_kernel_stats.csv"))))

    def med(which, kname, counter):
        path = os.path.join(outdir, "pmc_counted_%s" % which, "pmc_counter_collection.csv")
        v = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
             if kname in r["Kernel_Name"] and r["Counter_Name"] == counter]
        return statistics.median(v) if v else float("nan")

    md = ["# row_kernel, decode chains: bytes past the L2 and fabric read latency", "",
          "Commands (`$REPO` is the repository root, `$OUT` the output directory):", "",
          "    " + PROFILE_COMMANDS["trace_counted"], ""]
    for key, counters in DECODE_COUNTER_SETS.items():
        md.append("    " + PROFILE_COMMANDS["pmc_counted"].format(C=counters, N=key))
    md += ["", "Kernel source sha256[:16]: `%s`" % source_digest(), "",
           "Each chain is one row-kernel instance, captured in a graph of 160 calls "
           "(t = 8, d = 8192) and replayed; LL chains give every call its own words and flag "
           "(fresh from HBM), plain chains re-read one partial set. Under the profiler every "
           "dispatch runs alone, so durations are longer than in the untraced graphs and the "
           "caches see only one call at a time. Byte counters are medians per dispatch, scaled "
           "by the copy calibration (fetch x%.3f, write x%.3f). Latency: median over dispatches "
           "of the summed outstanding fabric read requests per cycle divided by the number of "
           "requests." % (kf, kw), "",
           "| chain | kernel | traced µs | algorithmic read / write bytes | fetched bytes | "
           "written bytes | fabric read latency (cycles) |", "|---|---|---|---|---|---|---|"]
    rec = {}
    for label in DECODE_COUNTED:
        sh = _counted_shape(label)
        kname = _counted_kernel(label)
        rd, wr = algorithmic_bytes(sh["n"], sh["t"], sh["d"], ll=sh["ll"])
        avg = [float(r["AverageNs"]) / 1e3 for r in rows if kname in r["Name"]]
        fb = med("fetch", kname, "FETCH_SIZE") * 1024 * kf
        wb = med("write", kname, "WRITE_SIZE") * 1024 * kw
        lat = med("lat", kname, "TCC_EA0_RDREQ_LEVEL_sum") / med("lat", kname, "TCC_EA0_RDREQ_sum")
        rec[label] = dict(kernel=kname, traced_us=avg[0] if avg else None, read=rd, write=wr,
                          fetched=fb, written=wb, read_latency_cycles=lat)
        md.append("| %s | `%s` | %s | %d / %d | %.0f | %.0f | %.0f |" % (
            label, kname, "%.2f" % avg[0] if avg else "?", rd, wr, fb, wb, lat))
    fl = [r for r in rows if "floor_kernel" in r["Name"]]
    if fl:
        md += ["", "The empty kernel of the same launches averages %.2f µs under this tracer." %
               (float(fl[0]["AverageNs"]) / 1e3)]
    with open(os.path.join(PROFILES, "row_kernel_decode_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(PROFILES, "row_kernel_decode_counters.json"), "w") as f:
        json.dump(dict(source_sha256_16=source_digest(), copy_factors=dict(fetch=kf, write=kw),
                       chains=rec), f, indent=1)
        f.write("\n")


# ------------------------------------------------------------ extras

def extra_table():
    """label -> zero-argument callable of every secondary measurement."""
    t = {"stream_copy_1GiB": stream_copy_gbps,
         "prefill_n8_t512_d8192": lambda: prefill_gbps(8, 512, 8192, 100, 10),
         "fp4_n4_t512_d8192": lambda: prefill_gbps(4, 512, 8192, 100, 10, fp4=True, out=False),
         # the same byte mixes without the arithmetic, in the calls' launch shapes
         "mix_9r2w_t512_d8192": lambda: mix_gbps(9, 2, 512, 8192, 100, 10),
         "mix_5r1w_t512_d8192": lambda: mix_gbps(5, 1, 512, 8192, 100, 10),
         "mix_9r2w_t4096_d8192": lambda: mix_gbps(9, 2, 4096, 8192, 30, 5),
         # wide rows (the kernel's chunk pipeline), same bytes as the timed workload
         "prefill_n8_t1024_d32768": lambda: prefill_gbps(8, 1024, 32768, 30, 5),
         "prefill_n8_t512_d65536": lambda: prefill_gbps(8, 512, 65536, 30, 5)}
    for label, out_, kw in [("allreduce_only_n8_t4096_d8192", True, dict(norm=False)),
                            ("fp8_n8_t4096_d8192", False, dict(fp8=True)),
                            ("no_residual_n8_t4096_d8192", True, dict(residual=False)),
                            ("sentinel_reset_n8_t4096_d8192", True, dict(reset=True))]:
        t[label] = (lambda out_=out_, kw=kw: prefill_gbps(8, 4096, 8192, 30, 5, out=out_, **kw))
    for (nn, tt, dd, kk, mode, fp4, label) in [
            (2, 1, 4096, 100, "", False, "decode_n2_t1_d4096_x100"),
            (8, 8, 4096, 64, "", False, "decode_n8_t8_d4096_chain64"),
            (4, 8, 8192, 160, "", False, "decode_n4_t8_d8192_chain160"),
            (8, 8, 8192, 160, "", False, "decode_n8_t8_d8192_chain160"),
            (4, 8, 8192, 160, "ll", False, "decode_n4_t8_d8192_chain160_ll"),
            (8, 8, 8192, 160, "ll", False, "decode_n8_t8_d8192_chain160_ll"),
            (8, 8, 8192, 160, "sentinel", False, "decode_n8_t8_d8192_chain160_sentinel"),
            (8, 8, 8192, 160, "fresh", False, "decode_n8_t8_d8192_chain160_fresh"),
            (8, 8, 8192, 160, "ll_reused", False, "decode_n8_t8_d8192_chain160_ll_reused"),
            (8, 8, 8192, 160, "sentinel_fresh", False, "decode_n8_t8_d8192_chain160_sentinel_fresh"),
            (8, 8, 8192, 160, "fp8", False, "decode_n8_t8_d8192_chain160_fp8"),
            (4, 1, 8192, 100, "", True, "fp4_n4_t1_d8192_x100"),
            (4, 8, 8192, 100, "", True, "fp4_n4_t8_d8192_x100"),
            (4, 64, 8192, 100, "", True, "fp4_n4_t64_d8192_x100"),
            # split rows: 2, 4 or 8 workgroups per row
            (4, 8, 8192, 160, "split4", False, "decode_n4_t8_d8192_chain160_split4"),
            (8, 8, 8192, 160, "split2", False, "decode_n8_t8_d8192_chain160_split2"),
            (8, 8, 8192, 160, "split4", False, "decode_n8_t8_d8192_chain160_split4"),
            (8, 8, 8192, 160, "split8", False, "decode_n8_t8_d8192_chain160_split8"),
            (8, 8, 8192, 160, "ll_split4", False, "decode_n8_t8_d8192_chain160_ll_split4"),
            (8, 8, 8192, 160, "sentinel_split4", False, "decode_n8_t8_d8192_chain160_sentinel_split4"),
            (8, 8, 8192, 160, "ll_split8", False, "decode_n8_t8_d8192_chain160_ll_split8"),
            (4, 8, 8192, 160, "ll_split8", False, "decode_n4_t8_d8192_chain160_ll_split8"),
            (8, 8, 8192, 160, "fresh_split4", False, "decode_n8_t8_d8192_chain160_fresh_split4"),
            (8, 8, 8192, 160, "sentinel_fresh_split4", False,
             "decode_n8_t8_d8192_chain160_sentinel_fresh_split4"),
            (8, 8, 8192, 160, "ll_reused_split8", False, "decode_n8_t8_d8192_chain160_ll_reused_split8"),
            (4, 1, 8192, 100, "split8", True, "fp4_n4_t1_d8192_x100_split8"),
            (4, 8, 8192, 100, "split4", True, "fp4_n4_t8_d8192_x100_split4"),
            (4, 64, 8192, 100, "split4", True, "fp4_n4_t64_d8192_x100_split4"),
            (8, 8, 8192, 160, "fp8_split8", False, "decode_n8_t8_d8192_chain160_fp8_split8"),
            # shapes where one workgroup per row leaves most of each CU's time to
            # a single row: twice the width, and 128 rows (two rows per CU)
            (8, 8, 16384, 100, "", False, "decode_n8_t8_d16384_x100"),
            (8, 8, 16384, 100, "split8", False, "decode_n8_t8_d16384_x100_split8"),
            (8, 128, 8192, 50, "", False, "decode_n8_t128_d8192_x50"),
            (8, 128, 8192, 50, "split2", False, "decode_n8_t128_d8192_x50_split2"),
            # the all-reduce alone (no norm, so no exchange when split)
            (8, 8, 8192, 160, "allreduce", False, "decode_n8_t8_d8192_chain160_allreduce"),
            (8, 8, 8192, 160, "allreduce_split8", False,
             "decode_n8_t8_d8192_chain160_allreduce_split8")]:
        sp = int(mode.split("split")[1]) if "split" in mode else 0
        t[label] = (lambda nn=nn, tt=tt, dd=dd, kk=kk, mode=mode, fp4=fp4, sp=sp:
                    decode_chain(nn, tt, dd, kk, ll=mode.startswith("ll"), fp4=fp4, out=not fp4,
                                 sentinel=mode.startswith("sentinel"), fp8=mode.startswith("fp8"),
                                 fresh=(True if "fresh" in mode else False if "reused" in mode
                                        else None), split=sp,
                                 norm=not mode.startswith("allreduce")))
    return t


def run_extras(only=None):
    import torch
    out = {}
    for label, fn in extra_table().items():
        if only and label not in only:
            continue
        log("extra %s" % label)
        out[label] = fn()
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ decode map

# The decode configurations of the workload definition: (label, n, t, d,
# calls per graph, LL layout, FP4 output). Each is timed with whole rows
# (one workgroup per row) and with the library's own split choice
# (ARFUSE_SPLIT_AUTO), against the same-length graph of the empty kernel of
# the same launch.
DECODE_MAP = [
    ("C1_n2_t1_d4096", 2, 1, 4096, 100, False, False),
    ("C2_n8_t8_d4096_chain64", 8, 8, 4096, 64, False, False),
    ("C3_n4_t8_d8192_chain160", 4, 8, 8192, 160, False, False),
    ("C3_n8_t8_d8192_chain160", 8, 8, 8192, 160, False, False),
    ("C3_n4_t8_d8192_chain160_ll", 4, 8, 8192, 160, True, False),
    ("C3_n8_t8_d8192_chain160_ll", 8, 8, 8192, 160, True, False),
    ("C5_n4_t1_d8192_fp4_x100", 4, 1, 8192, 100, False, True),
    ("C5_n4_t8_d8192_fp4_x100", 4, 8, 8192, 100, False, True),
    ("C5_n4_t64_d8192_fp4_x100", 4, 64, 8192, 100, False, True),
]


def decode_map(full: dict):
    """Compact per-config record (µs per call p50, the floor, their ratio;
    whole rows and the automatic split); the full records go to `full`."""
    import reduce_residual_rmsnorm_amd as arf
    out = {}
    for label, n, t, d, k, ll, fp4 in DECODE_MAP:
        log("decode %s" % label)
        kw = dict(ll=ll, fp4=fp4, out=not fp4)
        whole = decode_chain(n, t, d, k, split=0, **kw)
        full[label + "_whole"] = whole
        rec = {"floor_us": round(whole["floor_us_per_node_p50"], 3),
               "whole_us": round(whole["us_per_call_p50"], 3),
               "whole_x": round(whole["ratio_to_floor"], 3)}
        auto = decode_chain(n, t, d, k, split=arf.ARFUSE_SPLIT_AUTO, **kw)
        if auto["split"] > 1:
            full[label + "_auto"] = auto
            rec.update(split=auto["split"], split_floor_us=round(auto["floor_us_per_node_p50"], 3),
                       split_us=round(auto["us_per_call_p50"], 3),
                       split_x=round(auto["ratio_to_floor"], 3))
        else:
            rec.update(split=1)
        best = min([rec["whole_x"]] + ([rec["split_x"]] if "split_x" in rec else []))
        rec["best_x"] = best
        out[label] = rec
    return out


def prefill_t512(full: dict, steps: int = 100, warmup: int = 10):
    """The single-round prefill calls (t = 512: one round of workgroups) next
    to the same byte mix in the same launch shape without the arithmetic."""
    out = {}
    log("prefill t=512 (C4)")
    c4 = prefill_gbps(8, 512, 8192, steps, warmup)
    log("byte mix of C4 t=512: 9 planes read, 2 written")
    m4 = mix_gbps(9, 2, 512, 8192, steps, warmup)
    full["prefill_n8_t512_d8192"], full["mix_9r2w_t512_d8192"] = c4, m4
    out["C4_n8_t512_d8192"] = {
        "us": round(c4["us_per_call"], 2), "gbps_counted": round(c4["counted_gbps"], 1),
        "pct_counted": round(100 * c4["counted_gbps"] / PEAK_HBM_GBPS, 1),
        "gbps_alg": round(c4["algorithmic_gbps"], 1),
        "mix_us": round(m4["us_per_call"], 2), "mix_gbps": round(m4["gbps"], 1)}
    log("prefill t=512 FP4 (C5)")
    c5 = prefill_gbps(4, 512, 8192, steps, warmup, fp4=True, out=False)
    log("byte mix of C5 t=512: 5 planes read, 1 written")
    m5 = mix_gbps(5, 1, 512, 8192, steps, warmup)
    full["fp4_n4_t512_d8192"], full["mix_5r1w_t512_d8192"] = c5, m5
    out["C5_n4_t512_d8192_fp4"] = {
        "us": round(c5["us_per_call"], 2), "gbps_alg": round(c5["algorithmic_gbps"], 1),
        "mix_us": round(m5["us_per_call"], 2), "mix_gbps": round(m5["gbps"], 1)}
    return out


def reap_children(timeout_s: float = 30.0) -> int:
    """Wait for (then end) any child process still alive, so the benchmark
    exits with nothing of its own left running; returns how many there were."""
    try:
        import psutil
    except ImportError:
        return 0
    kids = psutil.Process().children(recursive=True)
    for k in kids:
        log("child process still alive at exit: pid %d %s" % (k.pid, " ".join(k.cmdline()[:4])))
    _, alive = psutil.wait_procs(kids, timeout=timeout_s)
    for k in alive:
        k.kill()
    psutil.wait_procs(alive, timeout=5)
    return len(kids)


def bench_record(name, n, t, d, steps, warmup, ms, ms_p50, value, achieved, traffic, cpu,
                 cpu_all, dec, t512):
    """The one JSON record bench.py prints last (kept to a few KB: the full
    records of every measurement go to the extras file)."""
    if cpu:
        cpu = dict(cpu, value=round(cpu["value"], 3))
    return {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_p50": round(ms_p50, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1)/sqrt(N) partials, N(0,1) residual with 0.1% x100 rows, "
                "U(0.5,1.5) gamma)",
        "config": {"workload": name, "n_partials": n, "tokens": t, "hidden": d,
                   "pct_of_peak_counted": round(100 * value / PEAK_HBM_GBPS, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "cpu_baseline_threads": ({"value": round(cpu_all["value"], 2), "unit": "GB/s",
                                  "cores": cpu_all["cores"]} if cpu_all else None),
        "decode": dec,
        "prefill_t512": t512,
        "kernel_source": source_digest(),
    }


# ------------------------------------------------------------ main

def build_if_missing() -> None:
    """Compile the HIP library in-tree when it has not been built (the
    benchmark runs what is built; it builds only when nothing is)."""
    pkg = os.path.join(os.path.dirname(os.path.abspath(__file__)), "reduce_residual_rmsnorm_amd")
    if os.path.exists(os.path.join(pkg, "lib", "libarfuse.so")):
        return
    import importlib.util
    spec = importlib.util.spec_from_file_location("arfuse_build", os.path.join(pkg, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    log("library not built: building %s" % mod.build())


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed prefill workload (no decode map, no t=512 figures)")
    ap.add_argument("--all-extras", action="store_true",
                    help="also run every secondary measurement (into --extras-out)")
    ap.add_argument("--extras-out", default=os.path.join("bench_out", "bench_extras.json"),
                    help="JSON file for the full records of every secondary measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-reps", type=int, default=200,
                    help="graph replays per decode measurement")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run the streaming-copy reference (counter calibration)")
    ap.add_argument("--only-extra", action="append", metavar="LABEL",
                    help="run only these secondary measurements (no timed workload) and "
                         "print them as one JSON object; repeatable")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 outputs under DIR, then exit")
    ap.add_argument("--profiles-dest", default=PROFILES,
                    help="directory the --summarize-profiles summaries are written to")
    args = ap.parse_args(argv)
    set_decode_reps(args.decode_reps)
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profiles_dest)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    build_if_missing()
    import reduce_residual_rmsnorm_amd as arf
    import seeded_inputs as si

    if args.copy_only:
        r = stream_copy_gbps()
        print(json.dumps(dict(stream_copy=r)), flush=True)
        return 0
    if args.only_extra:
        unknown = set(args.only_extra) - set(extra_table())
        if unknown:
            print("unknown extra(s): %s" % ", ".join(sorted(unknown)), file=sys.stderr)
            return 2
        print(json.dumps(dict(extras=run_extras(set(args.only_extra)),
                              kernel_source=source_digest())), flush=True)
        return 0

    name = "prefill_n8_t4096_d8192"
    log("generating %s" % name)
    ci = si.make_workload(name)
    n, t, d = ci.n, ci.t, ci.d
    rd, wr = algorithmic_bytes(n, t, d)
    sets = PrefillSets(ci, n_sets_for(rd + wr))
    info = arf.arfuse_query_launch(n, t, d, arf.ARFUSE_EPI_BF16)
    log("timing %d steps after %d warmup (%d rotating sets, grid %d x block %d)"
        % (args.steps, args.warmup, len(sets.sets), info.grid, info.block))
    ms = time_calls(sets.call, args.steps, args.warmup)
    value = counted_bytes(n, t, d) / (ms * 1e-3) / 1e9
    achieved = (rd + wr) / (ms * 1e-3) / 1e9
    # a second pass with an event between every call, for the median call
    each = time_calls_each(sets.call, args.steps, args.warmup + args.steps)
    ms_p50 = statistics.median(each)
    log("%.2f us/call (p50 %.2f), %.0f GB/s counted, %.0f GB/s algorithmic"
        % (ms * 1e3, ms_p50 * 1e3, value, achieved))
    del sets
    torch.cuda.empty_cache()

    full = {}
    dec = t512 = None
    if not args.no_extras:
        dec = decode_map(full)
        torch.cuda.empty_cache()
        t512 = prefill_t512(full)
        torch.cuda.empty_cache()
        if args.all_extras:
            full.update(run_extras())
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(ci)
        # the host's share of cores for one GPU is at most 16 threads
        threads = max(1, min(16, os.cpu_count() or 1))
        log("cpu baseline (oracle), rows on %d threads" % threads)
        cpu_all = cpu_baseline_threads(ci, threads)

    if full:
        try:
            os.makedirs(os.path.dirname(os.path.abspath(args.extras_out)), exist_ok=True)
            with open(args.extras_out, "w") as f:
                json.dump(dict(kernel_source=source_digest(), records=full), f, indent=1)
            log("full records written to %s" % args.extras_out)
        except OSError as e:
            log("could not write %s: %s" % (args.extras_out, e))
    for label, rec in (dec or {}).items():
        log("decode %s: %s" % (label, json.dumps(rec)))

    line = bench_record(name, n, t, d, args.steps, args.warmup, ms, ms_p50, value, achieved,
                        recorded_traffic(name), cpu, cpu_all, dec, t512)
    nkids = reap_children()
    if nkids:
        line["children_reaped"] = nkids
    print(json.dumps(line, separators=(",", ":")), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
