"""Fusion patterns beyond the default one, and the sentinel arrival layout,
against the oracle on the GPU.

Patterns (Deep Dive: AllReduce and AllReduce Fusion in TensorRT-LLM, §6.3):
no residual (h = the rank sum), all-reduce only (no gamma: residual_out is
the reduced tensor), no residual_out, FP8 output with or without the bf16
normalized output; in the plain and the LL layout.

Sentinel layout (the one-shot kernel's arrival test, Deep Dive §5.2, and the
sentinel mode of "Every µs Matters"): a 16-byte vector holding the sentinel
pattern has not arrived; it is re-read a bounded number of times and counted
into the status word if it never arrives; the call can refill a second slot
set with the sentinel (triple buffering clears the set two calls ahead).
The chain test replays a graph in which a copy node stands in for the peers'
push into slot set k % 3 before call k, and call k resets set (k + 2) % 3."""

import numpy as np
import pytest
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import (DEV, assert_fp4_close, assert_residual_exact, assert_y_close, dev_f32,
                      dev_u16, dev_u8, host_u16, note)

pytestmark = pytest.mark.gpu
LL = arf.ARFUSE_LAYOUT_LL
SENT = arf.ARFUSE_LAYOUT_SENTINEL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def orc():
    return __import__("oracle").default()


def new_status():
    return torch.zeros(4, dtype=torch.int32, device=DEV)


def read_status(st):
    v = st.cpu().numpy().view(np.uint32)
    return int(v[0]), int(v[2]) | (int(v[3]) << 32)


def assert_fp8_close(got, want, frac=1e-4):
    """FP8 codes: at most `frac` differ, each by one E4M3 step, same sign."""
    g = got.astype(np.int16)
    w = want.astype(np.int16)
    diff = g != w
    if diff.any():
        assert np.all((g[diff] & 0x80) == (w[diff] & 0x80)), "FP8 sign differs"
        assert np.abs((g[diff] & 0x7F) - (w[diff] & 0x7F)).max() <= 1, "FP8 off by more than a step"
    assert diff.sum() <= frac * g.size, "FP8: %d of %d codes differ" % (diff.sum(), g.size)
    return int(diff.sum())


def run(ci, *, residual=True, gamma=True, out=True, rout=True, fp4=False, fp8=None, layout=0,
        flag=None, **opts):
    """Run one call on the device with the requested pattern; returns host outputs."""
    t, d = ci.t, ci.d
    if layout == LL:
        parts = [dev_u8(si.ll_pack(p, flag)) for p in ci.partials]
    else:
        parts = [dev_u16(p) for p in ci.partials]
    res = dev_u16(ci.residual) if residual else None
    g = dev_f32(ci.gamma) if gamma else None
    o = torch.empty((t, d), dtype=torch.bfloat16, device=DEV) if out else None
    ro = torch.empty((t, d), dtype=torch.bfloat16, device=DEV) if rout else None
    codes = torch.empty((t, d // 2), dtype=torch.uint8, device=DEV) if fp4 else None
    scales = torch.empty((t, d // 16), dtype=torch.uint8, device=DEV) if fp4 else None
    f8 = torch.empty((t, d), dtype=torch.uint8, device=DEV) if fp8 is not None else None
    arf.arfuse_rmsnorm_ex(parts, res, g, float(ci.eps), o, ro, codes, scales, t=t, d=d,
                          layout=layout, ll_flag=flag or 0, fp8_out=f8,
                          fp8_inv_scale=fp8 if fp8 is not None else 1.0, **opts)
    torch.cuda.synchronize()
    return dict(residual_out=host_u16(ro) if rout else None, out=host_u16(o) if out else None,
                codes=codes.cpu().numpy() if fp4 else None,
                scales=scales.cpu().numpy() if fp4 else None,
                fp8=f8.cpu().numpy() if fp8 is not None else None)


PATTERNS = {
    "no_residual": dict(residual=False),
    "no_residual_fp4": dict(residual=False, out=False, fp4=True),
    "allreduce_only": dict(gamma=False, out=False),
    "allreduce_only_no_residual": dict(gamma=False, out=False, residual=False),
    "no_residual_out": dict(rout=False),
    "fp8": dict(out=False, fp8=1.0),
    "fp8_scaled_with_bf16": dict(fp8=37.5),
    "fp8_no_residual": dict(residual=False, out=False, fp8=0.25),
}


@pytest.mark.parametrize("layout", [0, LL, SENT])
@pytest.mark.parametrize("pattern", sorted(PATTERNS))
def test_pattern(pattern, layout):
    kw = PATTERNS[pattern]
    ci = si.make_call(8, 9, 8192, seed=60 + len(pattern), outlier_frac=0.2)
    flag = ci.ll_base + 1
    ref = orc().fused(ci.partials, ci.residual if kw.get("residual", True) else None,
                      ci.gamma if kw.get("gamma", True) else None, ci.eps,
                      out=kw.get("out", True), fp4=kw.get("fp4", False),
                      fp8_inv_scale=kw.get("fp8"), residual_out=kw.get("rout", True))
    note("pattern %s layout %d" % (pattern, layout))
    extra = dict(status=new_status(), max_polls=1) if layout in (LL, SENT) else {}
    got = run(ci, layout=layout, flag=flag, **kw, **extra)
    if extra:
        assert read_status(extra["status"]) == (0, 0)
    if kw.get("rout", True):
        assert_residual_exact(got["residual_out"], ref["residual_out"])
    if got["out"] is not None:
        assert_y_close(got["out"], ref["y32"], ref["out"])
    if got["codes"] is not None:
        assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
    if got["fp8"] is not None:
        assert_fp8_close(got["fp8"], ref["fp8"])


@pytest.mark.parametrize("n,t,d", [(1, 3, 16), (3, 5, 1040), (8, 64, 8192), (5, 2, 65536)])
def test_fp8_shapes(n, t, d):
    ci = si.make_call(n, t, d, seed=70 + n, outlier_frac=0.1)
    ref = orc().fused(ci.partials, ci.residual, ci.gamma, ci.eps, fp8_inv_scale=3.0)
    note("fp8 n=%d t=%d d=%d" % (n, t, d))
    got = run(ci, fp8=3.0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert assert_fp8_close(got["fp8"], ref["fp8"]) <= 1e-4 * ref["fp8"].size


# Rows wider than 16,384 elements: the kernel runs them as a pipeline of
# chunks with loads one or two chunks ahead; ragged widths leave idle lanes in
# the last chunk. (n, t, d, layout, outputs)
WIDE = [(8, 3, 32768, 0, dict()), (8, 2, 32768, LL, dict(fp4=True)),
        (8, 2, 65536, SENT, dict(fp8=2.0)), (3, 5, 40976, LL, dict(out=False, fp8=0.5)),
        (8, 4, 24592, SENT, dict(fp4=True)), (5, 2, 65520, 0, dict(fp4=True))]


@pytest.mark.parametrize("n,t,d,layout,kw", WIDE)
def test_wide_rows(n, t, d, layout, kw):
    ci = si.make_call(n, t, d, seed=90 + n, outlier_frac=0.3)
    ref = orc().fused(ci.partials, ci.residual, ci.gamma, ci.eps, out=kw.get("out", True),
                      fp4=kw.get("fp4", False), fp8_inv_scale=kw.get("fp8"))
    info = arf.arfuse_query_launch(n, t, d)
    note("wide n=%d t=%d d=%d layout=%d vpt=%d block=%d %s" % (n, t, d, layout, info.vpt,
                                                              info.block, kw))
    st = new_status()
    got = run(ci, layout=layout, flag=ci.ll_base + 3, status=st, max_polls=1, **kw)
    assert read_status(st) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    if got["out"] is not None:
        assert_y_close(got["out"], ref["y32"], ref["out"])
    if got["codes"] is not None:
        assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
    if got["fp8"] is not None:
        assert_fp8_close(got["fp8"], ref["fp8"])


# ------------------------------------------------------------ sentinel layout

def test_sentinel_complete_data_matches_plain():
    ci = si.make_workload("decode_n8_t8_d8192_chain160")
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True)
    st = new_status()
    note("sentinel complete")
    got = run(ci, fp4=True, layout=SENT, status=st, max_polls=2)
    assert read_status(st) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])


@pytest.mark.parametrize("sentinel", [0, 0xFFC1, 0x8000])
@pytest.mark.parametrize("max_polls", [0, 5])
def test_sentinel_pending_vectors_reported(sentinel, max_polls):
    ci = si.make_call(4, 6, 4096, seed=80)
    pat = sentinel or arf.ARFUSE_SENTINEL_DEFAULT
    for p in ci.partials:       # data never equals the pattern (producer side)
        p[p == pat] = 0
    ci.partials[1, 2, 17] = pat                # row 2
    ci.partials[1, 2, 18] = pat                # same vector: counts once
    ci.partials[3, 5, 4095] = pat              # row 5, last vector
    ci.partials[0, 5, 0:16] = pat              # row 5, two vectors
    pending = sum(orc().sentinel_pending(p, pat) for p in ci.partials)
    assert pending == 4
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    st = new_status()
    note("sentinel pending polls=%d pattern=%x" % (max_polls, pat))
    got = run(ci, layout=SENT, sentinel=sentinel, status=st, max_polls=max_polls)
    assert read_status(st) == (arf.ARFUSE_ERR_FLAG_TIMEOUT, pending)
    clean = [0, 1, 3, 4]
    assert_residual_exact(got["residual_out"][clean], ref["residual_out"][clean])
    assert_y_close(got["out"][clean], ref["y32"][clean])


# t <= 128: extra workgroups of the launch write the reset; above, every row
# workgroup refills its own row at its end.
# (2, 1024, 1024): a call of several workgroup rounds (the streaming-store
# instances) whose rows refill their own slots
@pytest.mark.parametrize("n,t,d", [(3, 5, 1040), (2, 128, 4096), (3, 129, 1040), (8, 300, 8192),
                                   (2, 1024, 1024)])
def test_sentinel_reset_refills_slots(n, t, d):
    ci = si.make_call(n, t, d, seed=81)
    info = arf.arfuse_query_launch(n, t, d, layout=SENT, reset=[1 << 32] * n)
    note("sentinel reset n=%d t=%d d=%d grid=%d" % (n, t, d, info.grid))
    parts = [dev_u16(p) for p in ci.partials]
    res = dev_u16(ci.residual)
    g = dev_f32(ci.gamma)
    o = torch.empty((t, d), dtype=torch.bfloat16, device=DEV)
    ro = torch.empty_like(o)
    slots = [torch.full((t, d), 7, dtype=torch.int16, device=DEV) for _ in range(n)]
    note("sentinel reset")
    st = new_status()
    arf.arfuse_rmsnorm_ex(parts, res, g, float(ci.eps), o, ro, layout=SENT, sentinel=0xFFC1,
                          reset=slots, status=st)
    torch.cuda.synchronize()
    assert read_status(st) == (0, 0)
    for sl in slots:
        assert np.all(sl.cpu().numpy().view(np.uint16) == 0xFFC1)
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    assert_residual_exact(host_u16(ro), ref["residual_out"])


@pytest.mark.parametrize("t", [9, 130])
def test_sentinel_allreduce_only_with_reset(t):
    """All-reduce only (no gamma) returns before the norm; the row workgroups'
    reset (t > 128) or the extra reset workgroups (t <= 128) must still run."""
    n, d = 4, 4096
    ci = si.make_call(n, t, d, seed=84)
    parts = [dev_u16(p) for p in ci.partials]
    ro = torch.empty((t, d), dtype=torch.bfloat16, device=DEV)
    slots = [torch.zeros((t, d), dtype=torch.int16, device=DEV) for _ in range(n)]
    note("sentinel all-reduce only with reset t=%d" % t)
    st = new_status()
    arf.arfuse_rmsnorm_ex(parts, dev_u16(ci.residual), None, float(ci.eps), None, ro, t=t, d=d,
                          layout=SENT, reset=slots, status=st)
    torch.cuda.synchronize()
    assert read_status(st) == (0, 0)
    for sl in slots:
        assert np.all(sl.cpu().numpy().view(np.uint16) == arf.ARFUSE_SENTINEL_DEFAULT)
    ref = orc().fused(ci.partials, ci.residual, None, ci.eps)
    assert_residual_exact(host_u16(ro), ref["residual_out"])


@pytest.mark.parametrize("layout", [SENT, LL])
def test_late_arrival_is_waited_for(layout):
    """A producer on a second stream spins for a few milliseconds, then copies
    the partials into the slots, while the fused call, already running on the
    current stream, re-reads them: it must see the data arrive (status clean)
    and produce the oracle's result on it. The LL slots start as words with
    the previous flag and a different payload, the sentinel slots as the
    pattern."""
    n, t, d = 4, 8, 4096
    ci = si.make_call(n, t, d, seed=95)
    flag = ci.ll_base + 7
    if layout == LL:
        data = [dev_u8(si.ll_pack(p, flag)) for p in ci.partials]
        slots = [dev_u8(si.ll_pack(np.zeros_like(p), flag - 1)) for p in ci.partials]
    else:
        data = [dev_u16(p) for p in ci.partials]
        slots = [torch.full((t, d), -1, dtype=torch.int16, device=DEV) for _ in range(n)]
    res = dev_u16(ci.residual)
    g = dev_f32(ci.gamma)
    o = torch.empty((t, d), dtype=torch.bfloat16, device=DEV)
    ro = torch.empty_like(o)
    st = new_status()
    producer = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("late arrival layout %d" % layout)
    with torch.cuda.stream(producer):
        torch.cuda._sleep(10_000_000)
        for i in range(n):
            arf.arfuse_stream_copy(slots[i], data[i])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    arf.arfuse_rmsnorm_ex(slots, res, g, float(ci.eps), o, ro, t=t, d=d, layout=layout,
                          ll_flag=flag, max_polls=1_000_000, status=st)
    e1.record()
    torch.cuda.synchronize()
    waited_ms = e0.elapsed_time(e1)
    note("late arrival: the call took %.3f ms" % waited_ms)
    assert waited_ms > 0.1, "the call did not wait: the test did not exercise the re-reads"
    assert read_status(st) == (0, 0)
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    assert_residual_exact(host_u16(ro), ref["residual_out"])
    assert_y_close(host_u16(o), ref["y32"], ref["out"])


@pytest.mark.parametrize("split", [0, 4])
def test_sentinel_triple_buffered_chain_in_graph(split):
    n, t, d, k = 4, 8, 4096, 12
    ci = si.make_call(n, t, d, seed=82)
    sets = si.make_partial_sets(n, t, d, k, seed=83)
    sets[sets == arf.ARFUSE_SENTINEL_DEFAULT] = 0
    data = dev_u16(sets)                                   # [k][n][t][d]: what peers push
    slots = torch.full((3, n, t, d), -1, dtype=torch.int16, device=DEV)   # 0xFFFF
    res0 = dev_u16(ci.residual)
    bufs = [torch.empty_like(res0), torch.empty_like(res0)]
    g = dev_f32(ci.gamma)
    outs = torch.empty((k, t, d), dtype=torch.bfloat16, device=DEV)
    st = new_status()
    plane = t * d * 2
    ws = torch.zeros(256 * ((t + 7) // 8 * 8), dtype=torch.uint8, device=DEV) if split else None

    def enqueue():
        for c in range(k):
            cur, nxt = c % 3, (c + 2) % 3
            for i in range(n):   # the peers' push into this call's slot set
                arf.arfuse_stream_copy(slots[cur, i], data[c, i], plane)
            rin = res0 if c == 0 else bufs[c % 2]
            arf.arfuse_rmsnorm_ex([slots[cur, i] for i in range(n)], rin, g, float(ci.eps),
                                  outs[c], bufs[(c + 1) % 2], layout=SENT, max_polls=4,
                                  status=st, reset=[slots[nxt, i] for i in range(n)],
                                  split=split, workspace=ws)

    ref = orc().chain(sets, ci.residual, ci.gamma, ci.eps, k, per_call=True)
    note("sentinel chain split=%d eager" % split)
    enqueue()
    torch.cuda.synchronize()
    assert read_status(st) == (0, 0)
    assert_residual_exact(host_u16(bufs[k % 2]), ref[-1]["residual_out"])
    # the last two calls refilled the two sets the next calls would read
    for s in ((k + 1) % 3, (k + 0) % 3):
        assert np.all(slots[s].cpu().numpy().view(np.uint16) == 0xFFFF), "set %d not reset" % s
    gr = torch.cuda.CUDAGraph()
    note("sentinel chain split=%d capture" % split)
    with torch.cuda.graph(gr):
        enqueue()
    for rep in range(3):
        outs.zero_()
        bufs[0].zero_()
        bufs[1].zero_()
        st.zero_()
        torch.cuda.synchronize()
        note("sentinel chain split=%d replay %d" % (split, rep))
        gr.replay()
        torch.cuda.synchronize()
        assert read_status(st) == (0, 0)
        assert_residual_exact(host_u16(bufs[k % 2]), ref[-1]["residual_out"])
        oh = host_u16(outs)
        for c in range(k):
            assert_y_close(oh[c], ref[c]["y32"])
        enqueue()           # eager work between replays
        torch.cuda.synchronize()


# Calls whose rows take several rounds of workgroups (t * vpt >= 1536) run
# the instances that write their outputs through to memory (streaming
# stores); every output kind goes through them here, in the plain and the
# sentinel layout, and in a wide row (four vectors per thread).
STREAM_PATTERNS = {
    "bf16": dict(),
    "fp4": dict(out=False, fp4=True),
    "bf16_fp4": dict(fp4=True),
    "fp8": dict(out=False, fp8=2.0),
    "bf16_fp8": dict(fp8=0.5),
    "allreduce_only": dict(gamma=False, out=False),
    "no_residual": dict(residual=False),
}


@pytest.mark.parametrize("layout", [0, SENT])
@pytest.mark.parametrize("pattern", sorted(STREAM_PATTERNS))
def test_streaming_store_instances(pattern, layout):
    kw = STREAM_PATTERNS[pattern]
    n, t, d = 3, 1536, 1024
    epi = ((arf.ARFUSE_EPI_BF16 if kw.get("out", True) and kw.get("gamma", True) else 0)
           | (arf.ARFUSE_EPI_FP4 if kw.get("fp4") else 0)
           | (arf.ARFUSE_EPI_FP8 if kw.get("fp8") is not None else 0))
    assert arf.arfuse_query_launch(n, t, d, epi, layout=layout).stream_stores == 1
    assert arf.arfuse_query_launch(n, 512, d, epi, layout=layout).stream_stores == 0
    ci = si.make_call(n, t, d, seed=110 + len(pattern), outlier_frac=0.01)
    ref = orc().fused(ci.partials, ci.residual if kw.get("residual", True) else None,
                      ci.gamma if kw.get("gamma", True) else None, ci.eps,
                      out=kw.get("out", True), fp4=kw.get("fp4", False),
                      fp8_inv_scale=kw.get("fp8"))
    note("streaming stores %s layout %d t=%d d=%d" % (pattern, layout, t, d))
    extra = dict(status=new_status(), max_polls=1) if layout in (LL, SENT) else {}
    got = run(ci, layout=layout, **kw, **extra)
    if extra:
        assert read_status(extra["status"]) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    if got["out"] is not None:
        assert_y_close(got["out"], ref["y32"], ref["out"])
    if got["codes"] is not None:
        assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
    if got["fp8"] is not None:
        assert_fp8_close(got["fp8"], ref["fp8"])


def test_streaming_store_wide_rows():
    n, t, d = 2, 384, 32768
    info = arf.arfuse_query_launch(n, t, d, arf.ARFUSE_EPI_BF16 | arf.ARFUSE_EPI_FP4)
    assert info.vpt == 4 and info.stream_stores == 1
    ci = si.make_call(n, t, d, seed=120, outlier_frac=0.01)
    ref = orc().fused(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True)
    note("streaming stores wide rows t=%d d=%d" % (t, d))
    got = run(ci, fp4=True)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
