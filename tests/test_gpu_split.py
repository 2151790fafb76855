"""Split rows against the oracle on the GPU.

A row's columns are divided among 2, 4 or 8 workgroups. Each sums the squares
of its slice, publishes the share tagged with its dispatch's token in its slot
of a caller workspace (never cleared) and waits, bounded, for the row's other
shares; all of them add the shares in slice order. This is a re-layout of the row
reduction the fused operator does inside one workgroup (Deep Dive: AllReduce
and AllReduce Fusion in TensorRT-LLM, §6.3 and §6.5: RMSNorm over the whole
hidden dimension), so the outputs meet the same bar as the unsplit call:
residual_out bit-exact, y, FP4 and FP8 to the oracle's tolerance."""

import numpy as np
import pytest
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import (DEV, assert_fp4_close, assert_residual_exact, assert_y_close, dev_f32,
                      dev_u8, dev_u16, host_u16, note)

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
    """(code, exchange_timeouts, bad_words) of an arfuse_ll_status."""
    v = st.cpu().numpy().view(np.uint32)
    return int(v[0]), int(v[1]), int(v[2]) | (int(v[3]) << 32)


def padded(t):
    """Row positions of a split launch: t rounded up to a multiple of 8."""
    return (t + 7) // 8 * 8


def workspace(t, split):
    return torch.zeros(256 * padded(t), dtype=torch.uint8, device=DEV)


def active_slots(t, split):
    """16-byte slot indices the real rows write: row r's slices fill line r
    (8 slots) of each of the two regions of padded(t) lines."""
    return ([r * 8 + s for r in range(t) for s in range(split)] +
            [padded(t) * 8 + r * 8 + s for r in range(t) for s in range(split)])


def assert_fp8_close(got, want, frac=1e-4):
    g = got.astype(np.int16)
    w = want.astype(np.int16)
    diff = g != w
    if diff.any():
        assert np.all((g[diff] & 0x80) == (w[diff] & 0x80)), "FP8 sign differs"
        assert np.abs((g[diff] & 0x7F) - (w[diff] & 0x7F)).max() <= 1, "FP8 off by more than a step"
    assert diff.sum() <= frac * g.size, "FP8: %d of %d codes differ" % (diff.sum(), g.size)


class Call:
    """Device buffers of one call; `go` enqueues it with the given options."""

    def __init__(self, ci, *, layout=0, flag=None, residual=True, gamma=True, out=True,
                 rout=True, fp4=False, fp8=None):
        t, d = ci.t, ci.d
        self.ci, self.layout, self.flag, self.fp8 = ci, layout, flag, fp8
        if layout == LL:
            self.parts = [dev_u8(si.ll_pack(p, flag)) for p in ci.partials]
        else:
            self.parts = [dev_u16(p) for p in ci.partials]
        self.res = dev_u16(ci.residual) if residual else None
        self.g = dev_f32(ci.gamma) if gamma else None
        self.o = torch.empty((t, d), dtype=torch.bfloat16, device=DEV) if out else None
        self.ro = torch.empty((t, d), dtype=torch.bfloat16, device=DEV) if rout else None
        self.codes = torch.empty((t, d // 2), dtype=torch.uint8, device=DEV) if fp4 else None
        self.scales = torch.empty((t, d // 16), dtype=torch.uint8, device=DEV) if fp4 else None
        self.f8 = torch.empty((t, d), dtype=torch.uint8, device=DEV) if fp8 is not None else None

    def go(self, **opts):
        ci = self.ci
        arf.arfuse_rmsnorm_ex(self.parts, self.res, self.g, float(ci.eps), self.o, self.ro,
                              self.codes, self.scales, t=ci.t, d=ci.d, layout=self.layout,
                              ll_flag=self.flag or 0, fp8_out=self.f8,
                              fp8_inv_scale=self.fp8 if self.fp8 is not None else 1.0, **opts)

    def fetch(self):
        torch.cuda.synchronize()
        return dict(residual_out=host_u16(self.ro) if self.ro is not None else None,
                    out=host_u16(self.o) if self.o is not None else None,
                    codes=self.codes.cpu().numpy() if self.codes is not None else None,
                    scales=self.scales.cpu().numpy() if self.scales is not None else None,
                    fp8=self.f8.cpu().numpy() if self.f8 is not None else None)


def check(got, ref, rows=slice(None)):
    if got["residual_out"] is not None:
        assert_residual_exact(got["residual_out"][rows], ref["residual_out"][rows])
    if got["out"] is not None:
        assert_y_close(got["out"][rows], ref["y32"][rows], ref["out"][rows])
    if got["codes"] is not None:
        assert_fp4_close(got["codes"][rows], got["scales"][rows], ref["codes"][rows],
                         ref["scales"][rows])
    if got["fp8"] is not None:
        assert_fp8_close(got["fp8"][rows], ref["fp8"][rows])


def reference(ci, residual=True, gamma=True, out=True, rout=True, fp4=False, fp8=None):
    return orc().fused(ci.partials, ci.residual if residual else None,
                       ci.gamma if gamma else None, ci.eps, out=out, fp4=fp4,
                       fp8_inv_scale=fp8, residual_out=rout)


@pytest.mark.parametrize("split", [2, 4, 8])
@pytest.mark.parametrize("layout", [0, LL, SENT])
def test_split_matches_oracle(layout, split):
    ci = si.make_call(8, 9, 8192, seed=200 + split + 10 * layout, outlier_frac=0.2)
    flag = ci.ll_base + 5
    ref = reference(ci, fp4=True)
    c = Call(ci, layout=layout, flag=flag, fp4=True)
    st = new_status()
    info = arf.arfuse_query_launch(8, 9, 8192, arf.ARFUSE_EPI_BF16 | arf.ARFUSE_EPI_FP4,
                                   split=split, layout=layout)
    note("split %d layout %d grid %d block %d" % (split, layout, info.grid, info.block))
    c.go(split=split, workspace=workspace(9, split), status=st, max_polls=1)
    got = c.fetch()
    assert read_status(st) == (0, 0, 0)
    check(got, ref)


# ragged slices (idle lanes in the last vector group of each slice), the
# largest t * split, the widest row, the narrowest slice (16 elements)
SHAPES = [(3, 5, 2080, 2, dict(fp8=0.75)), (5, 7, 4160, 4, dict(fp4=True)),
          (2, 3, 1152, 8, dict()), (8, 32, 8192, 8, dict(fp4=True)),
          (5, 2, 65536, 8, dict(fp8=2.0)), (1, 1, 128, 8, dict(fp4=True)),
          (4, 64, 8192, 4, dict(fp4=True, out=False)), (7, 128, 3072, 2, dict())]


@pytest.mark.parametrize("n,t,d,split,kw", SHAPES)
def test_split_shapes(n, t, d, split, kw):
    ci = si.make_call(n, t, d, seed=210 + n + split, outlier_frac=0.3)
    ref = reference(ci, **kw)
    c = Call(ci, **kw)
    st = new_status()
    info = arf.arfuse_query_launch(n, t, d, split=split)
    note("split shape n=%d t=%d d=%d split=%d grid=%d block=%d %s"
         % (n, t, d, split, info.grid, info.block, kw))
    c.go(split=split, workspace=workspace(t, split), status=st)
    got = c.fetch()
    assert read_status(st) == (0, 0, 0)
    check(got, ref)


PATTERNS = {
    "no_residual": dict(residual=False),
    "no_residual_out": dict(rout=False),
    "fp8_no_residual": dict(residual=False, out=False, fp8=0.25),
    # no norm: nothing to exchange, no workspace needed
    "allreduce_only": dict(gamma=False, out=False),
}


@pytest.mark.parametrize("pattern", sorted(PATTERNS))
def test_split_patterns(pattern):
    kw = PATTERNS[pattern]
    ci = si.make_call(8, 9, 8192, seed=230 + len(pattern), outlier_frac=0.2)
    ref = reference(ci, **kw)
    c = Call(ci, **kw)
    ws = None if pattern == "allreduce_only" else workspace(9, 4)
    st = new_status()
    note("split pattern %s" % pattern)
    c.go(split=4, workspace=ws, status=st)
    check(c.fetch(), ref)
    assert read_status(st) == (0, 0, 0)


def test_split_sentinel_pending_and_reset():
    """Sentinel layout with split rows: a pending vector is counted once by the
    slice that holds it, the other rows are exact, and the reset refills the
    whole set (here by the launch's extra workgroups, t <= 128)."""
    n, t, d, split = 4, 6, 4096, 4
    ci = si.make_call(n, t, d, seed=240)
    pat = arf.ARFUSE_SENTINEL_DEFAULT
    for p in ci.partials:
        p[p == pat] = 0
    ci.partials[2, 3, 1030] = pat          # row 3, slice 1
    pending = sum(orc().sentinel_pending(p, pat) for p in ci.partials)
    assert pending == 1
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    c = Call(ci, layout=SENT)
    slots = [torch.zeros((t, d), dtype=torch.int16, device=DEV) for _ in range(n)]
    st = new_status()
    note("split sentinel pending + reset")
    c.go(split=split, workspace=workspace(t, split), status=st, max_polls=3, reset=slots)
    got = c.fetch()
    assert read_status(st) == (arf.ARFUSE_ERR_FLAG_TIMEOUT, 0, pending)
    clean = [0, 1, 2, 4, 5]
    check(got, ref, rows=clean)
    for sl in slots:
        assert np.all(sl.cpu().numpy().view(np.uint16) == pat)


def slot_tokens(ws, t, split):
    """The 64-bit tokens of the slots of the real rows."""
    w = ws.cpu().numpy().view(np.uint32).reshape(-1, 4)[active_slots(t, split)]
    return w[:, 2].astype(np.uint64) | (w[:, 3].astype(np.uint64) << np.uint64(32))


def test_split_tokens_over_calls_and_graph_replays():
    """Each slice tags its slot with a token of the kernel dispatch: eager
    calls and a captured chain replayed several times, with eager calls
    between the replays, all on one workspace; every call's outputs are the
    same bits (the shares are added in a fixed order), every slot of a call
    carries that call's one token, and no two calls share a token."""
    n, t, d, split, k = 8, 8, 8192, 4, 6
    ci = si.make_call(n, t, d, seed=250, outlier_frac=0.01)
    ref = reference(ci, fp4=True)
    c = Call(ci, fp4=True)
    ws = workspace(t, split)
    st = new_status()
    note("split tokens eager")
    c.go(split=split, workspace=ws, status=st)
    first = c.fetch()
    check(first, ref)
    seen = set()
    tok = slot_tokens(ws, t, split)
    assert len(set(tok.tolist())) == 1 and int(tok[0]) & (1 << 32), tok
    seen.add(int(tok[0]))

    def enqueue():
        for _ in range(k):
            c.go(split=split, workspace=ws, status=st)

    gr = torch.cuda.CUDAGraph()
    note("split tokens capture")
    with torch.cuda.graph(gr):
        enqueue()
    for rep in range(3):
        c.o.zero_()
        c.codes.zero_()
        torch.cuda.synchronize()
        note("split tokens replay %d" % rep)
        gr.replay()
        got = c.fetch()
        assert read_status(st) == (0, 0, 0)
        for key in ("residual_out", "out", "codes", "scales"):
            assert np.array_equal(got[key], first[key]), key
        tok = slot_tokens(ws, t, split)
        assert len(set(tok.tolist())) == 1 and int(tok[0]) not in seen, (rep, tok)
        seen.add(int(tok[0]))
        enqueue()
        torch.cuda.synchronize()
        tok = slot_tokens(ws, t, split)
        assert len(set(tok.tolist())) == 1 and int(tok[0]) not in seen, (rep, tok)
        seen.add(int(tok[0]))


def test_split_ignores_stale_workspace_contents():
    """The slots need no clearing: a workspace filled with garbage, one that
    still holds every slot of the previous call (its shares and its token),
    and one workspace reused by calls of different t and split with nothing
    cleared in between all give the oracle's outputs and a clean status."""
    n = 4
    shapes = [(3, 4096, 2), (8, 8192, 8), (5, 4096, 4), (8, 8192, 4), (1, 2048, 8), (3, 4096, 2)]
    ws = torch.full((256 * 8,), 0xA5, dtype=torch.uint8, device=DEV)   # garbage
    st = new_status()
    for i, (t, d, split) in enumerate(shapes):
        ci = si.make_call(n, t, d, seed=260 + i)
        ref = reference(ci, fp4=True)
        c = Call(ci, fp4=True)
        note("split stale workspace: t=%d d=%d split=%d" % (t, d, split))
        c.go(split=split, workspace=ws, status=st)
        check(c.fetch(), ref)
        assert read_status(st) == (0, 0, 0)
        # the same call again, every slot still holding this call's
        # predecessor: a stale share must not be taken for a fresh one
        saved = ws.clone()
        c.o.zero_()
        c.go(split=split, workspace=ws, status=st)
        check(c.fetch(), ref)
        assert read_status(st) == (0, 0, 0)
        assert not torch.equal(saved[:256 * padded(t)], ws[:256 * padded(t)])


# ARFUSE_SPLIT_AUTO: the library's choice for the shape, and the workspace
# that choice needs (one chosen split of each size, and one shape it leaves
# unsplit, which needs no workspace)
AUTO = [(8, 8, 8192, 0, dict(fp4=True)), (8, 128, 8192, 0, dict()), (8, 8, 4096, LL, dict()),
        (8, 8, 16384, SENT, dict(fp8=1.5)), (8, 8, 4096, 0, dict()),
        (8, 8, 4096, 0, dict(gamma=False, out=False)), (4, 8, 8192, SENT, dict(gamma=False, out=False))]


@pytest.mark.parametrize("n,t,d,layout,kw", AUTO)
def test_auto_split_matches_oracle(n, t, d, layout, kw):
    ci = si.make_call(n, t, d, seed=270 + t + layout, outlier_frac=0.2)
    ref = reference(ci, **kw)
    epi = 0 if not kw.get("gamma", True) else arf.ARFUSE_EPI_BF16
    info = arf.arfuse_query_launch(n, t, d, epi, layout=layout, split=arf.ARFUSE_SPLIT_AUTO)
    c = Call(ci, layout=layout, flag=ci.ll_base + 9, **kw)
    ws = workspace(t, info.split) if info.split > 1 else None
    st = new_status()
    note("auto split n=%d t=%d d=%d layout=%d -> split %d grid %d block %d"
         % (n, t, d, layout, info.split, info.grid, info.block))
    for _ in range(2):
        c.go(split=arf.ARFUSE_SPLIT_AUTO, workspace=ws, status=st, max_polls=1)
        check(c.fetch(), ref)
    assert read_status(st) == (0, 0, 0)


def test_split_residual_in_place():
    """residual_out may be the residual buffer itself: each slice reads its
    own columns of the residual before it writes them."""
    n, t, d, split = 8, 8, 8192, 8
    ci = si.make_call(n, t, d, seed=280, outlier_frac=0.2)
    ref = reference(ci, fp4=True)
    c = Call(ci, fp4=True)
    c.ro = c.res                 # in place
    st = new_status()
    note("split in-place residual")
    c.go(split=split, workspace=workspace(t, split), status=st)
    check(c.fetch(), ref)
    assert read_status(st) == (0, 0, 0)
