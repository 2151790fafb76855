"""A seeded sweep of valid call configurations against the oracle on the GPU.

Each case draws a rank count, a shape, an input layout (plain, LL,
sentinel), a fusion pattern (Deep Dive: AllReduce and AllReduce Fusion in
TensorRT-LLM, §6.3: all-reduce only, bf16 norm output, FP4 or FP8 with or
without it, with or without the residual and the residual output) and a row
split (none, 2, 4, 8 or automatic), then checks every output to the same
bar as the other parity tests. The draws are fixed by the seed, so a failing
case is reproduced by its test id."""

import numpy as np
import pytest
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import DEV, note
from test_gpu_split import Call, check, new_status, read_status, reference

pytestmark = pytest.mark.gpu
LL = arf.ARFUSE_LAYOUT_LL
SENT = arf.ARFUSE_LAYOUT_SENTINEL
AUTO = arf.ARFUSE_SPLIT_AUTO

PATTERNS = [dict(gamma=False, out=False), dict(), dict(out=False, fp4=True), dict(fp4=True),
            dict(out=False, fp8=0.5), dict(fp8=3.0)]
MAX_ELEMS = 3_000_000   # n * t * d per case: the oracle stays well under a second


def draw(case: int):
    rng = np.random.default_rng(7000 + case)
    n = int(rng.integers(1, 9))
    layout = int(rng.choice([0, LL, SENT]))
    kw = dict(PATTERNS[int(rng.integers(len(PATTERNS)))])
    kw["residual"] = bool(rng.random() < 0.8)
    norm = kw.get("gamma", True)
    if norm and rng.random() < 0.15:
        kw["rout"] = False
    split = int(rng.choice([0, 2, 4, 8, AUTO]))
    s = split if split in (2, 4, 8) else 1
    t = int(rng.integers(1, 256 // (8 if split == AUTO else s) + 1))
    t = min(t, 24)
    kmax = max(1, min(65536 // (16 * s), 16384 // 16 if s > 1 else 4096,
                      MAX_ELEMS // (n * t * 16 * s)))
    d = 16 * s * int(rng.integers(1, kmax + 1))
    return n, t, d, layout, split, kw


CASES = list(range(160))


@pytest.mark.parametrize("case", CASES)
def test_sweep_case(case):
    n, t, d, layout, split, kw = draw(case)
    ci = si.make_call(n, t, d, seed=7100 + case, outlier_frac=0.3)
    ref = reference(ci, **kw)
    flag = ci.ll_base + case
    c = Call(ci, layout=layout, flag=flag, **kw)
    opts = dict(status=new_status(), max_polls=1)
    if split:
        info = arf.arfuse_query_launch(n, t, d, layout=layout, split=split)
        opts.update(split=split, workspace=(torch.zeros(info.workspace_bytes, dtype=torch.uint8,
                                                        device=DEV)
                                            if info.workspace_bytes else None))
        eff = info.split
    else:
        eff = 1
    note("sweep case %d: n=%d t=%d d=%d layout=%d split=%d (runs %d) %s"
         % (case, n, t, d, layout, split, eff, kw))
    for _ in range(2):          # the second call finds the first call's slots stale
        c.go(**opts)
        check(c.fetch(), ref)
    assert read_status(opts["status"]) == (0, 0, 0)


def test_sweep_covers_the_space():
    """The draws reach every layout, every pattern, every split choice, rank
    counts at both ends and both residual choices (host only)."""
    drawn = [draw(c) for c in CASES]
    assert {x[3] for x in drawn} == {0, LL, SENT}
    assert {x[4] for x in drawn} == {0, 2, 4, 8, AUTO}
    assert {x[0] for x in drawn} >= {1, 8}
    pats = {tuple(sorted((k, v) for k, v in x[5].items() if k not in ("residual", "rout")))
            for x in drawn}
    assert len(pats) == len(PATTERNS)
    assert {x[5]["residual"] for x in drawn} == {True, False}
