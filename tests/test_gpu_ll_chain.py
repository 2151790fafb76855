"""LL-packed input decode and hipGraph-captured decode chains, vs the oracle.

LL: every 16-byte word carries 8 bytes of payload and an 8-byte flag; the
kernel checks each flag against the expected one, re-reads a mismatch at most
max_polls times and reports words that never matched in a device status word
(stale and corrupted flags are staged on the host before upload, so the
kernel always finishes).

Chains: K calls captured in one graph, call k reading call k-1's
residual_out (residual buffers ping-pong), as the cross-layer fusion of a
decode step chains them. The graph is replayed several times with eager work
and synchronizations in between; every replay is checked: final residual bit
exact against the oracle replaying the same K calls, every call's y within
tolerance."""

import numpy as np
import pytest
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import (DEV, Dev, assert_fp4_close, assert_residual_exact, assert_y_close, dev_f32,
                      dev_u16, dev_u8, host_u16, note)

pytestmark = pytest.mark.gpu

LL = arf.ARFUSE_LAYOUT_LL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def orc():
    return __import__("oracle").default()


def new_status():
    return torch.zeros(4, dtype=torch.int32, device=DEV)  # arfuse_ll_status, 16 bytes


def read_status(st):
    v = st.cpu().numpy().view(np.uint32)
    return int(v[0]), int(v[2]) | (int(v[3]) << 32)


def oracle_ll(ci, words_host, flag):
    """Oracle on LL words: unpack (counting bad flags), then the fused call."""
    parts, bad = [], 0
    for w in words_host:
        p, b = orc().ll_unpack(w, ci.t * ci.d, flag)
        parts.append(p.reshape(ci.t, ci.d))
        bad += b
    return orc().allreduce_rmsnorm(parts, ci.residual, ci.gamma, ci.eps, fp4=True), bad


@pytest.mark.parametrize("name", ["decode_n4_t8_d8192_chain160", "decode_n8_t8_d8192_chain160"])
@pytest.mark.parametrize("max_polls", [0, 8])
def test_ll_good_flags(name, max_polls):
    ci = si.make_workload(name)
    flag = ci.ll_base
    words = si.ll_pack_all(ci.partials, flag)
    ref, bad = oracle_ll(ci, words, flag)
    assert bad == 0
    dv = Dev(ci, fp4=True, ll_flag=flag)
    st = new_status()
    note("LL good flags %s polls=%d" % (name, max_polls))
    got = dv.run(layout=LL, ll_flag=flag, max_polls=max_polls, status=st).fetch()
    assert read_status(st) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])


@pytest.mark.parametrize("max_polls", [0, 3, 64])
def test_ll_stale_words_reported(max_polls):
    ci = si.make_call(8, 8, 8192, seed=21)
    flag = ci.ll_base + 5
    words = si.ll_pack_all(ci.partials, flag)
    # three stale words (the previous step's flag) in rows 1 and 6, ranks 0, 3, 7
    wpr = ci.d // 4
    si.ll_set_flag(words[0], [1 * wpr + 3], flag - 1)
    si.ll_set_flag(words[3], [1 * wpr + 2047], flag - 1)
    si.ll_set_flag(words[7], [6 * wpr + 1000], flag - 1)
    ref, bad = oracle_ll(ci, words, flag)
    assert bad == 3
    dv = Dev(ci, fp4=True)
    dv.parts = [dev_u8(w) for w in words]
    st = new_status()
    note("LL stale words polls=%d" % max_polls)
    got = dv.run(layout=LL, ll_flag=flag, max_polls=max_polls, status=st).fetch()
    code, nbad = read_status(st)
    assert code == arf.ARFUSE_ERR_FLAG_TIMEOUT and nbad == 3
    clean = [r for r in range(ci.t) if r not in (1, 6)]
    assert_residual_exact(got["residual_out"][clean], ref["residual_out"][clean])
    assert_y_close(got["out"][clean], ref["y32"][clean])


def test_ll_corrupted_partial_counts_every_word():
    ci = si.make_call(4, 2, 1024, seed=22)
    flag = ci.ll_base
    words = si.ll_pack_all(ci.partials, flag)
    words[2] = si.ll_pack(ci.partials[2], flag ^ 0xDEADBEEF)
    _, bad = oracle_ll(ci, words, flag)
    assert bad == ci.t * ci.d // 4
    dv = Dev(ci)
    dv.parts = [dev_u8(w) for w in words]
    st = new_status()
    note("LL corrupted partial")
    dv.run(layout=LL, ll_flag=flag, max_polls=2, status=st).fetch()
    assert read_status(st) == (arf.ARFUSE_ERR_FLAG_TIMEOUT, bad)


def test_ll_wide_row_vpt2():
    ci = si.make_call(3, 3, 16384, seed=23)
    flag = ci.ll_base
    words = si.ll_pack_all(ci.partials, flag)
    ref, _ = oracle_ll(ci, words, flag)
    dv = Dev(ci, fp4=True, ll_flag=flag)
    st = new_status()
    note("LL d=16384")
    got = dv.run(layout=LL, ll_flag=flag, status=st).fetch()
    assert read_status(st) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])


# ----------------------------------------------------------------- chains

class Chain:
    """K chained calls over device buffers; capture into a graph or run eagerly."""

    def __init__(self, n, t, d, k, seed, per_call_sets=False, ll=False, split=0):
        self.n, self.t, self.d, self.k = n, t, d, k
        self.split = split
        # split rows: one workspace for every call of the chain, zeroed once
        self.ws = (torch.zeros(256 * ((t + 7) // 8 * 8), dtype=torch.uint8, device=DEV)
                   if split > 1
                   else None)
        ci = si.make_call(n, t, d, seed=seed)
        self.ci = ci
        self.flags = [ci.ll_base + c for c in range(k)]
        self.ll = ll
        if per_call_sets:
            self.sets = si.make_partial_sets(n, t, d, k, seed + 1)
        else:
            self.sets = None
        if ll:
            packed = np.stack([si.ll_pack_all(self.sets[c], self.flags[c]) for c in range(k)])
            self.parts_dev = dev_u8(packed)          # [k][n][t][d/4][16]
            self.words_host = packed
        elif per_call_sets:
            self.parts_dev = dev_u16(self.sets)       # [k][n][t][d]
        else:
            self.parts_dev = dev_u16(ci.partials)     # [n][t][d]
        self.res0 = dev_u16(ci.residual)
        self.bufs = [torch.empty_like(self.res0), torch.empty_like(self.res0)]
        self.gamma = dev_f32(ci.gamma)
        self.outs = torch.empty((k, t, d), dtype=torch.bfloat16, device=DEV)
        self.status = new_status()

    def parts(self, c):
        if self.ll or self.sets is not None:
            return [self.parts_dev[c, i] for i in range(self.n)]
        return [self.parts_dev[i] for i in range(self.n)]

    def enqueue(self):
        for c in range(self.k):
            rin, rout = self.bufs[c % 2], self.bufs[(c + 1) % 2]
            rin = self.res0 if c == 0 else rin
            if self.ll:
                arf.arfuse_rmsnorm_ex(self.parts(c), rin, self.gamma, self.ci.eps, self.outs[c], rout,
                                      layout=LL, ll_flag=self.flags[c], max_polls=4,
                                      status=self.status, split=self.split, workspace=self.ws)
            elif self.split:
                arf.arfuse_rmsnorm_ex(self.parts(c), rin, self.gamma, self.ci.eps, self.outs[c], rout,
                                      status=self.status, split=self.split, workspace=self.ws)
            else:
                arf.arfuse_rmsnorm(self.parts(c), rin, self.gamma, self.ci.eps, self.outs[c], rout)

    def final(self):
        return self.bufs[self.k % 2]

    def oracle(self):
        if self.ll:
            sets = []
            for c in range(self.k):
                ps = []
                for i in range(self.n):
                    p, bad = orc().ll_unpack(self.words_host[c, i], self.t * self.d, self.flags[c])
                    assert bad == 0
                    ps.append(p.reshape(self.t, self.d))
                sets.append(np.stack(ps))
            return orc().chain(sets, self.ci.residual, self.ci.gamma, self.ci.eps, self.k,
                               per_call=True)
        src = self.sets if self.sets is not None else self.ci.partials
        return orc().chain(src, self.ci.residual, self.ci.gamma, self.ci.eps, self.k,
                           per_call=self.sets is not None)


def check_chain(ch, ref, what):
    torch.cuda.synchronize()
    assert_residual_exact(host_u16(ch.final()), ref[-1]["residual_out"], what + " final residual")
    outs = host_u16(ch.outs)
    for c in range(ch.k):
        assert_y_close(outs[c], ref[c]["y32"])
    if ch.ll or ch.split:
        assert read_status(ch.status) == (0, 0)
        assert int(ch.status.cpu().numpy().view(np.uint32)[1]) == 0, "exchange timeouts"


@pytest.mark.parametrize("n,t,d,k,per_call,ll", [
    (8, 8, 4096, 64, False, False),      # Llama-3-8B decode step: 32 layers x 2
    (4, 8, 8192, 160, False, False),     # Llama-3.1-70B decode step: 80 layers x 2
    (8, 8, 8192, 160, False, False),
    (8, 8, 8192, 160, True, True),       # LL, one partial set and flag per call
    (4, 8, 8192, 160, True, True),
])
def test_graph_chain(n, t, d, k, per_call, ll):
    ch = Chain(n, t, d, k, seed=30 + n, per_call_sets=per_call, ll=ll)
    ref = ch.oracle()
    what = "chain n=%d d=%d k=%d ll=%s" % (n, d, k, ll)
    note(what + " eager")
    ch.enqueue()
    check_chain(ch, ref, what + " eager")
    g = torch.cuda.CUDAGraph()
    note(what + " capture")
    with torch.cuda.graph(g):
        ch.enqueue()
    for rep in range(3):
        ch.outs.zero_()
        ch.bufs[0].zero_()
        ch.bufs[1].zero_()
        ch.status.zero_()
        torch.cuda.synchronize()
        note(what + " replay %d" % rep)
        g.replay()
        check_chain(ch, ref, what + " replay %d" % rep)
        # eager work between replays
        ch.enqueue()
        torch.cuda.synchronize()


@pytest.mark.parametrize("n,t,d,k,per_call,ll,split", [
    (8, 8, 8192, 160, False, False, 4),
    (8, 8, 8192, 160, True, False, 8),   # fresh partials per call
    (8, 8, 8192, 160, True, True, 8),    # LL, one partial set and flag per call
    (4, 8, 4096, 64, False, False, 2),
])
def test_graph_chain_split_rows(n, t, d, k, per_call, ll, split):
    """The same chains with split rows: every call's slices find each other's
    shares by the call's own token, in eager runs and graph replays alike."""
    ch = Chain(n, t, d, k, seed=40 + n, per_call_sets=per_call, ll=ll, split=split)
    ref = ch.oracle()
    what = "split chain n=%d d=%d k=%d ll=%s split=%d" % (n, d, k, ll, split)
    note(what + " eager")
    ch.enqueue()
    check_chain(ch, ref, what + " eager")
    g = torch.cuda.CUDAGraph()
    note(what + " capture")
    with torch.cuda.graph(g):
        ch.enqueue()
    for rep in range(3):
        ch.outs.zero_()
        ch.bufs[0].zero_()
        ch.bufs[1].zero_()
        ch.status.zero_()
        torch.cuda.synchronize()
        note(what + " replay %d" % rep)
        g.replay()
        check_chain(ch, ref, what + " replay %d" % rep)
        ch.enqueue()
        torch.cuda.synchronize()
    pt = (t + 7) // 8 * 8      # row positions; line r of each region holds row r's slots
    w = ch.ws.cpu().numpy().view(np.uint32).reshape(2 * pt * 8, 4)
    w = w[[reg * pt * 8 + r * 8 + s for reg in range(2) for r in range(t) for s in range(split)]]
    tok = w[:, 2].astype(np.uint64) | (w[:, 3].astype(np.uint64) << np.uint64(32))
    assert len(set(tok.tolist())) == 1 and int(tok[0]) & (1 << 32), \
        "every slot carries the last call's token"


@pytest.mark.parametrize("n,t,d", [(3, 5, 48), (5, 7, 1040), (6, 3, 8208), (2, 2, 65520),
                                   (8, 9, 4112), (1, 4, 16)])
def test_ll_ragged_shapes(n, t, d):
    ci = si.make_call(n, t, d, seed=40 + n + d, outlier_frac=0.2)
    flag = ci.ll_base + 3
    words = si.ll_pack_all(ci.partials, flag)
    ref, bad = oracle_ll(ci, words, flag)
    assert bad == 0
    dv = Dev(ci, fp4=True, ll_flag=flag)
    st = new_status()
    note("LL ragged n=%d t=%d d=%d" % (n, t, d))
    got = dv.run(layout=LL, ll_flag=flag, max_polls=1, status=st).fetch()
    assert read_status(st) == (0, 0)
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"], ref["out"])
    assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"])
