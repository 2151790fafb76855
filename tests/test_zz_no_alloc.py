"""The allocation-free entry point (arfuse_rmsnorm_noalloc) against the
workspace entry point (arfuse_rmsnorm_ex) through the C ABI: the same
kernels, with the split rows' exchange slots in the library's static array
instead of a caller workspace, so the outputs must be the same bits. Two
calls in a row, the second smaller; a captured chain; and the argument
rules of the entry point."""

import numpy as np
import pytest
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import (DEV, assert_fp4_close, assert_residual_exact, assert_y_close, dev_f32,
                      dev_u8, dev_u16, host_u16, note)

pytestmark = pytest.mark.gpu
LL = arf.ARFUSE_LAYOUT_LL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def orc():
    return __import__("oracle").default()


class Bufs:
    """Device inputs of one call and two output sets: one for each entry."""

    def __init__(self, ci, layout=0, flag=0):
        t, d = ci.t, ci.d
        self.ci, self.layout, self.flag = ci, layout, flag
        if layout == LL:
            self.parts = [dev_u8(si.ll_pack(p, flag)) for p in ci.partials]
        else:
            self.parts = [dev_u16(p) for p in ci.partials]
        self.res = dev_u16(ci.residual)
        self.g = dev_f32(ci.gamma)
        self.outs = [dict(o=torch.empty((t, d), dtype=torch.bfloat16, device=DEV),
                          ro=torch.empty((t, d), dtype=torch.bfloat16, device=DEV),
                          codes=torch.empty((t, d // 2), dtype=torch.uint8, device=DEV),
                          scales=torch.empty((t, d // 16), dtype=torch.uint8, device=DEV),
                          st=torch.zeros(4, dtype=torch.int32, device=DEV))
                     for _ in range(2)]

    def call(self, which, split, noalloc, ws=None):
        b, ci = self.outs[which], self.ci
        kw = dict(t=ci.t, d=ci.d, layout=self.layout, ll_flag=self.flag, max_polls=1,
                  status=b["st"], split=split)
        args = (self.parts, self.res, self.g, float(ci.eps), b["o"], b["ro"], b["codes"],
                b["scales"])
        if noalloc:
            arf.arfuse_rmsnorm_noalloc(*args, **kw)
        else:
            arf.arfuse_rmsnorm_ex(*args, workspace=ws, **kw)

    def host(self, which):
        b = self.outs[which]
        return dict(out=host_u16(b["o"]), residual_out=host_u16(b["ro"]),
                    codes=b["codes"].cpu().numpy(), scales=b["scales"].cpu().numpy(),
                    status=b["st"].cpu().numpy().view(np.uint32).copy())


def workspace_for(n, t, d, layout, split):
    info = arf.arfuse_query_launch(n, t, d, arf.ARFUSE_EPI_BF16 | arf.ARFUSE_EPI_FP4,
                                   layout=layout, split=split)
    return info, (torch.zeros(int(info.workspace_bytes), dtype=torch.uint8, device=DEV)
                  if info.workspace_bytes else None)


def same_as_workspace_entry(ci, split, layout=0):
    """One call through each entry on the same inputs: identical bits, clean
    status, and the oracle's bar."""
    flag = ci.ll_base + 11
    bufs = Bufs(ci, layout, flag)
    info, ws = workspace_for(ci.n, ci.t, ci.d, layout, split)
    note("noalloc vs workspace entry: n=%d t=%d d=%d layout=%d split=%s (runs %d)"
         % (ci.n, ci.t, ci.d, layout, split, info.split))
    bufs.call(0, split, noalloc=False, ws=ws)
    bufs.call(1, split, noalloc=True)
    torch.cuda.synchronize()
    want, got = bufs.host(0), bufs.host(1)
    for key in ("residual_out", "out", "codes", "scales"):
        assert np.array_equal(got[key], want[key]), key
    assert not got["status"].any() and not want["status"].any(), (got["status"], want["status"])
    ref = orc().allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
    return info.split


def test_two_calls_in_a_row_the_second_smaller():
    """The largest split call the slots hold (t * split = 256), then a smaller
    one on the same slots, then a smaller LL one: each equal to the workspace
    entry's bits."""
    big = si.make_call(8, 32, 8192, seed=300, outlier_frac=0.1)
    assert same_as_workspace_entry(big, 8) == 8
    small = si.make_call(4, 3, 4096, seed=301)
    assert same_as_workspace_entry(small, 4) == 4
    ll = si.make_call(8, 2, 8192, seed=302)
    assert same_as_workspace_entry(ll, arf.ARFUSE_SPLIT_AUTO, layout=LL) == 8


def test_decode_shapes_with_the_automatic_split():
    for (n, t, d) in [(8, 8, 8192), (4, 1, 8192), (4, 64, 8192), (2, 1, 4096)]:
        same_as_workspace_entry(si.make_call(n, t, d, seed=310 + t), arf.ARFUSE_SPLIT_AUTO)


def test_captured_chain_replays():
    """A chain captured in a graph (call c takes call c-1's residual_out),
    after a t = 0 call that looks the slots up outside the capture; three
    replays, with eager calls of another shape between them, each equal to
    the same chain through the workspace entry."""
    n, t, d, k = 8, 8, 8192, 12
    ci = si.make_call(n, t, d, seed=320, outlier_frac=0.1)
    parts = [dev_u16(p) for p in ci.partials]
    res0 = dev_u16(ci.residual)
    g = dev_f32(ci.gamma)
    arf.arfuse_rmsnorm_noalloc(parts, None, g, float(ci.eps), None, None, t=0, d=d)

    def make():
        return dict(bufs=[torch.empty_like(res0), torch.empty_like(res0)],
                    outs=torch.empty((k, t, d), dtype=torch.bfloat16, device=DEV),
                    st=torch.zeros(4, dtype=torch.int32, device=DEV))

    def enqueue(b, noalloc, ws=None):
        for c in range(k):
            rin = res0 if c == 0 else b["bufs"][c % 2]
            args = (parts, rin, g, float(ci.eps), b["outs"][c], b["bufs"][(c + 1) % 2])
            if noalloc:
                arf.arfuse_rmsnorm_noalloc(*args, status=b["st"], split=arf.ARFUSE_SPLIT_AUTO)
            else:
                arf.arfuse_rmsnorm_ex(*args, status=b["st"], split=arf.ARFUSE_SPLIT_AUTO,
                                      workspace=ws)

    info, ws = workspace_for(n, t, d, 0, arf.ARFUSE_SPLIT_AUTO)
    assert info.split > 1
    want = make()
    note("noalloc chain: workspace entry, eager")
    enqueue(want, False, ws)
    torch.cuda.synchronize()
    got = make()
    gr = torch.cuda.CUDAGraph()
    note("noalloc chain: capture")
    with torch.cuda.graph(gr):
        enqueue(got, True)
    other = si.make_call(4, 3, 4096, seed=321)
    for rep in range(3):
        got["outs"].zero_()
        got["bufs"][0].zero_()
        got["bufs"][1].zero_()
        torch.cuda.synchronize()
        note("noalloc chain: replay %d" % rep)
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(got["outs"]), host_u16(want["outs"])), rep
        assert np.array_equal(host_u16(got["bufs"][k % 2]), host_u16(want["bufs"][k % 2])), rep
        assert not got["st"].cpu().numpy().any()
        same_as_workspace_entry(other, 4)      # other calls on the same slots in between


def test_argument_rules():
    """A workspace is refused (the static slots replace it); a split beyond
    the slots is refused as by the workspace entry; a split call without a
    status word is refused; t = 0 is a no-op."""
    ci = si.make_call(4, 33, 4096, seed=330)   # buffers hold every t requested below
    parts = [dev_u16(p) for p in ci.partials]
    res, g = dev_u16(ci.residual), dev_f32(ci.gamma)
    o, ro = torch.empty_like(res), torch.empty_like(res)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    ws = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    lib = arf.lib
    import ctypes
    arr = (ctypes.c_void_p * 4)(*[p.data_ptr() for p in parts])

    def call(t, d, **opts):
        op = arf._opts(**opts)
        return lib.arfuse_rmsnorm_noalloc(arr, 4, res.data_ptr(), g.data_ptr(), 1e-5,
                                          o.data_ptr(), ro.data_ptr(), None, None, t, d, 0,
                                          ctypes.byref(op))

    assert call(1, 4096, split=2, status=st.data_ptr(),
                workspace=ws.data_ptr()) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(33, 4096, split=8, status=st.data_ptr()) == arf.ARFUSE_ERR_UNSUPPORTED
    assert call(1, 4096, split=2) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(0, 4096, split=8) == arf.ARFUSE_OK
