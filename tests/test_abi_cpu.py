"""C-ABI library: loads, exports every declared symbol, and validates its
arguments on the host before any HIP call (no GPU needed: every call here
either returns an argument error or is a t == 0 no-op)."""

import ctypes
import math
import os
import re

import pytest

import reduce_residual_rmsnorm_amd as arf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arfuse.h")

# fake, 16-byte aligned, never dereferenced device addresses
A = [0x10000 * (i + 1) for i in range(16)]
T, D = 8, 4096
PLANE = T * D * 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(arfuse_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(arf.EXPORTED)


@pytest.mark.parametrize("name", sorted(arf.EXPORTED))
def test_symbol_exported(name):
    lib = ctypes.CDLL(arf.LIB_PATH)
    assert hasattr(lib, name)


def test_version_and_status_strings():
    assert arf.arfuse_version() == 4
    for code in range(5):
        assert arf.arfuse_status_string(code)
    assert arf.arfuse_status_string(99) == "unknown status"


def call(parts=None, n=None, residual=None, gamma=None, eps=1e-5, out=None, residual_out=None,
         fp4=None, scales=None, t=T, d=D, opts=None):
    parts = list(A[:4]) if parts is None else parts
    n = len(parts) if n is None else n
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts else None
    args = [arr, n, A[8] * 16 if residual is None else residual,
            A[9] * 16 if gamma is None else gamma, eps,
            A[10] * 16 if out is None else out,
            A[11] * 16 if residual_out is None else residual_out, fp4 or 0, scales or 0, t, d, 0]
    if opts is None:
        return arf.lib.arfuse_rmsnorm(*args)
    return arf.lib.arfuse_rmsnorm_ex(*args, ctypes.byref(opts))


BIG = 1 << 32  # spacing that keeps the fake buffers of a [8][4096] call apart


def spaced(i):
    return BIG * (i + 1)


def good(**kw):
    base = dict(parts=[spaced(i) for i in range(4)], residual=spaced(8), gamma=spaced(9),
                out=spaced(10), residual_out=spaced(11))
    base.update(kw)
    return base


INVALID = {
    "no_partials_array": dict(parts=[], n=1),
    "n_zero": dict(n=0),
    "n_nine": dict(parts=[spaced(i) for i in range(9)]),
    "null_partial": dict(parts=[spaced(0), 0]),
    "misaligned_partial": dict(parts=[spaced(0) + 8]),
    "null_gamma": dict(gamma=0),
    "misaligned_out": dict(out=spaced(10) + 4),
    "fp4_without_scales": dict(fp4=spaced(12)),
    "scales_without_fp4": dict(scales=spaced(13)),
    "negative_t": dict(t=-1),
    "zero_d": dict(d=0),
    "d_not_multiple_of_16": dict(d=4104),
    "negative_eps": dict(eps=-1e-5),
    "nan_eps": dict(eps=float("nan")),
    "inf_eps": dict(eps=float("inf")),
    "out_is_partial": dict(out=spaced(1)),
    "residual_out_is_partial": dict(residual_out=spaced(2)),
    "out_is_residual": dict(out=spaced(8)),
    "out_overlaps_residual_out": dict(out=spaced(11) + PLANE - 16),
    "residual_out_overlaps_residual": dict(residual_out=spaced(8) + 16),
    "out_overlaps_gamma": dict(out=spaced(9) - PLANE + 16),
    "fp4_overlaps_out": dict(fp4=spaced(10) + 16, scales=spaced(13)),
    "scales_overlap_fp4": dict(fp4=spaced(12), scales=spaced(12) + 16),
    "norm_output_without_gamma": dict(gamma=0),
    "allreduce_without_residual_out": dict(gamma=0, out=0, residual_out=0),
    "misaligned_residual": dict(residual=spaced(8) + 2),
    "nothing_to_write": dict(out=0, residual_out=0),
}


@pytest.mark.parametrize("case", sorted(INVALID))
def test_invalid_arguments_rejected(case):
    assert call(**good(**INVALID[case])) == arf.ARFUSE_ERR_INVALID_ARG


def test_patterns_accepted_at_t_zero_and_rejected_when_inconsistent():
    # all-reduce only: no gamma, no norm outputs, residual_out present
    assert call(**good(gamma=0, out=0, t=0)) == arf.ARFUSE_OK
    # no residual, norm outputs only
    assert call(**good(residual=0, residual_out=0, t=0)) == arf.ARFUSE_OK
    # FP8 options
    o = arf._opts(fp8_out=spaced(13), fp8_inv_scale=float("inf"))
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(fp8_out=spaced(13), fp8_inv_scale=2.0)
    assert call(**good(fp4=spaced(12), scales=spaced(14), opts=o)) == arf.ARFUSE_ERR_UNSUPPORTED
    o = arf._opts(fp8_out=spaced(10) + 16, fp8_inv_scale=2.0)   # overlaps out
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG


def test_sentinel_options_validated():
    S = arf.ARFUSE_LAYOUT_SENTINEL
    assert call(**good(opts=arf._opts(layout=3))) == arf.ARFUSE_ERR_INVALID_ARG
    # reset buffers only with the sentinel layout
    o = arf._opts(reset=[spaced(20 + i) for i in range(4)])
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(layout=S, sentinel=0x1FFFF)
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    # a reset buffer overlapping a partial, or missing
    o = arf._opts(layout=S, reset=[spaced(0)] + [spaced(21 + i) for i in range(3)])
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(layout=S, reset=[0] + [spaced(21 + i) for i in range(3)])
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(layout=S, reset=[spaced(20 + i) for i in range(4)])
    assert call(**good(opts=o, t=0)) == arf.ARFUSE_OK
    o = arf._opts()
    o.reserved2 = 1
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    # the re-read bound
    o = arf._opts(layout=S, max_polls=arf.ARFUSE_MAX_POLLS)
    assert call(**good(opts=o, t=0)) == arf.ARFUSE_OK
    o = arf._opts(layout=S, max_polls=arf.ARFUSE_MAX_POLLS + 1)
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG


def test_unsupported_width():
    assert call(**good(d=65536 + 16)) == arf.ARFUSE_ERR_UNSUPPORTED


def test_t_zero_is_a_noop():
    assert call(**good(t=0)) == arf.ARFUSE_OK
    # buffers may be NULL (an empty tensor's data pointer) when t == 0
    assert call(parts=[0, 0], residual=0, gamma=0, out=0, residual_out=0, t=0) == arf.ARFUSE_OK
    assert call(**good(t=0, eps=-1.0)) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(**good(t=0, d=24)) == arf.ARFUSE_ERR_INVALID_ARG


def test_bad_options_rejected():
    o = arf._opts(layout=7)
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    for bt in (32, 100, 2048):
        assert call(**good(opts=arf._opts(block_threads=bt))) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(**good(opts=arf._opts(vpt=3))) == arf.ARFUSE_ERR_INVALID_ARG
    # an override that cannot cover the row
    assert call(**good(opts=arf._opts(block_threads=64, vpt=1))) == arf.ARFUSE_ERR_UNSUPPORTED


def test_ll_partials_occupy_twice_the_bytes():
    # plain partials one plane apart are fine; as LL they overlap each other's
    # successor... only outputs are checked against inputs, so place out one
    # plane after a partial: valid for plain, overlapping for LL.
    kw = good(out=spaced(0) + PLANE)
    assert call(**dict(kw, t=0)) == arf.ARFUSE_OK
    o = arf._opts(layout=arf.ARFUSE_LAYOUT_LL, status=spaced(30))
    assert call(**dict(kw, opts=o)) == arf.ARFUSE_ERR_INVALID_ARG


def test_waiting_calls_need_a_status_word():
    """A call that can wait (LL or sentinel arrival, a split row's exchange)
    reports a bounded wait that gave up only in its status word, so without
    one it is refused before anything is enqueued. (With one, the same calls
    pass validation: checked in the sanitized host build, which stops at an
    empty kernel selector instead of launching.)"""
    INV = arf.ARFUSE_ERR_INVALID_ARG
    ws = spaced(40)
    for o in (arf._opts(layout=arf.ARFUSE_LAYOUT_LL), arf._opts(layout=arf.ARFUSE_LAYOUT_SENTINEL),
              arf._opts(split=4, workspace=ws), arf._opts(split=arf.ARFUSE_SPLIT_AUTO, workspace=ws)):
        assert call(**good(opts=o, d=8192)) == INV
        assert call(**good(opts=o, d=8192, t=0)) == arf.ARFUSE_OK   # t = 0 stays a no-op
    # the automatic choice above does split at this shape
    assert arf.arfuse_query_launch(4, T, 8192, split=arf.ARFUSE_SPLIT_AUTO).split > 1


@pytest.mark.parametrize("d,block,vpt", [(16, 64, 1), (4096, 512, 1), (8192, 1024, 1),
                                         (8208, 576, 2), (16384, 1024, 2), (65536, 1024, 8),
                                         (48, 64, 1)])
def test_query_launch_auto(d, block, vpt):
    info = arf.arfuse_query_launch(8, 5, d)
    assert (info.grid, info.block, info.vpt) == (5, block, vpt)
    assert info.block * info.vpt * 8 >= d


@pytest.mark.parametrize("n,t,d,extra", [(8, 8, 8192, 8 * 8), (3, 5, 1040, 3 * 4), (2, 128, 4096, 2 * 128),
                                         (3, 129, 1040, 0), (8, 4096, 8192, 0)])
def test_query_launch_sentinel_reset_blocks(n, t, d, extra):
    """Up to 128 rows, n * ceil(t*d/8 / block) reset workgroups follow the rows."""
    S = arf.ARFUSE_LAYOUT_SENTINEL
    info = arf.arfuse_query_launch(n, t, d, layout=S, reset=[spaced(i) for i in range(n)])
    base = arf.arfuse_query_launch(n, t, d, layout=S)
    assert base.grid == t
    assert info.grid == t + extra
    if extra:
        assert extra == n * -(-(t * d // 8) // info.block)


def test_query_launch_override():
    info = arf.arfuse_query_launch(8, 3, 8192, block_threads=512)
    assert (info.block, info.vpt) == (512, 2)
    info = arf.arfuse_query_launch(8, 3, 8192, vpt=4)
    assert (info.block, info.vpt) == (256, 4)


def test_quantize_and_copy_validation():
    q = arf.lib.arfuse_quantize_fp4
    assert q(spaced(0), 4, 4104, spaced(1), spaced(2), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert q(spaced(0) + 4, 4, 4096, spaced(1), spaced(2), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert q(spaced(0), 4, 4096, spaced(0) + 16, spaced(2), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert q(0, 4, 4096, spaced(1), spaced(2), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert q(spaced(0), 0, 4096, spaced(1), spaced(2), 0) == arf.ARFUSE_OK
    assert q(0, 0, 4096, 0, 0, 0) == arf.ARFUSE_OK
    c = arf.lib.arfuse_stream_copy
    assert c(spaced(0), spaced(1), 24, 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert c(spaced(0), spaced(0) + 16, 64, 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert c(spaced(0), spaced(1), 0, 0) == arf.ARFUSE_OK
    for r, vec in ((arf.lib.arfuse_round_bf16, 2), (arf.lib.arfuse_round_fp8, 4)):
        assert r(spaced(0), vec + 1, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG   # not a multiple
        assert r(spaced(0), -vec, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG
        assert r(0, vec, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG
        assert r(spaced(0), 4 * vec, spaced(0) + 4, 0) == arf.ARFUSE_ERR_INVALID_ARG  # overlap
        assert r(spaced(0), 0, 0, 0) == arf.ARFUSE_OK
    assert arf.lib.arfuse_round_fp8(spaced(0) + 8, 4, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG
    r4 = arf.lib.arfuse_round_fp4
    assert r4(spaced(0), 3, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG     # odd
    assert r4(spaced(0), -2, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert r4(0, 2, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG
    assert r4(spaced(0) + 4, 2, spaced(1), 0) == arf.ARFUSE_ERR_INVALID_ARG  # 8-byte alignment
    assert r4(spaced(0), 8, spaced(0) + 4, 0) == arf.ARFUSE_ERR_INVALID_ARG  # overlap
    assert r4(spaced(0), 0, 0, 0) == arf.ARFUSE_OK


def test_single_hip_runtime_in_process():
    """Importing the binding first must not leave two HIP runtimes in the
    process (PyTorch carries its own libamdhip64 under the same soname)."""
    import subprocess
    import sys
    code = ("import reduce_residual_rmsnorm_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       check=True)
    assert r.stdout.strip() == "1", r.stdout + r.stderr


def test_binding_rejects_host_small_and_strided_tensors():
    """The binding checks tensors before the C call: a host tensor's address
    would make the kernel fault, a short or strided one would be read past its
    end or in the wrong order. (Raw int addresses are passed through.)"""
    import torch
    t, d = 2, 64
    cpu = torch.zeros(t, d, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        arf.arfuse_rmsnorm([cpu], cpu, torch.ones(d), 1e-5, cpu, cpu)
    with pytest.raises(ValueError, match="GPU tensor"):
        arf.arfuse_stream_copy(torch.zeros(16, dtype=torch.uint8), torch.zeros(16, dtype=torch.uint8))

    class FakeCuda:
        """A stand-in for a GPU tensor (no GPU here): shape facts only."""
        def __init__(self, nbytes, contiguous=True):
            self.is_cuda, self._n, self._c, self.device = True, nbytes, contiguous, "cuda:0"
            self.shape = (t, d)
        def is_contiguous(self):
            return self._c
        def numel(self):
            return self._n
        def element_size(self):
            return 1
        def data_ptr(self):
            return spaced(50)

    plane = t * d * 2
    ok = FakeCuda(plane)
    with pytest.raises(ValueError, match="holds 255 bytes"):
        arf.arfuse_rmsnorm([FakeCuda(plane - 1)], ok, FakeCuda(4 * d), 1e-5, ok, FakeCuda(plane))
    with pytest.raises(ValueError, match="contiguous"):
        arf.arfuse_rmsnorm([ok], ok, FakeCuda(4 * d), 1e-5, FakeCuda(plane, contiguous=False), ok)
    with pytest.raises(ValueError, match="partials\\[0\\] holds"):   # LL words are twice the bytes
        arf.arfuse_rmsnorm_ex([FakeCuda(plane)], ok, FakeCuda(4 * d), 1e-5, ok, ok,
                              layout=arf.ARFUSE_LAYOUT_LL)
    with pytest.raises(ValueError, match="status"):
        arf.arfuse_rmsnorm_ex([ok], ok, FakeCuda(4 * d), 1e-5, ok, ok, status=FakeCuda(8))


def test_split_options_validated():
    """split must be 1, 2, 4 or 8, divide the row in whole FP4 blocks, keep
    t * split within the resident cap and come with an aligned workspace that
    overlaps no other buffer."""
    ws = spaced(40)
    assert call(**good(opts=arf._opts(split=4, workspace=ws), t=0)) == arf.ARFUSE_OK
    for bad_split in (3, 16):
        assert call(**good(opts=arf._opts(split=bad_split, workspace=ws))) == arf.ARFUSE_ERR_INVALID_ARG
    # 4112 = 16 * 257: whole FP4 blocks per slice only without a split
    assert call(**good(opts=arf._opts(split=2, workspace=ws), d=4112)) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(**good(opts=arf._opts(split=4))) == arf.ARFUSE_ERR_INVALID_ARG  # no workspace
    assert call(**good(opts=arf._opts(split=4, workspace=ws + 8))) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(**good(opts=arf._opts(split=8, workspace=ws), t=33)) == arf.ARFUSE_ERR_UNSUPPORTED
    # slices wider than 16,384 elements, or more than 2 vectors per thread
    assert call(**good(opts=arf._opts(split=2, workspace=ws), d=65536, t=1)) == arf.ARFUSE_ERR_UNSUPPORTED
    assert call(**good(opts=arf._opts(split=4, vpt=4, workspace=ws), d=8192)) == arf.ARFUSE_ERR_UNSUPPORTED
    # the workspace is written: it may overlap neither a partial nor an output
    assert call(**good(opts=arf._opts(split=2, workspace=spaced(0)))) == arf.ARFUSE_ERR_INVALID_ARG
    assert call(**good(opts=arf._opts(split=2, workspace=spaced(11) + 16))) == arf.ARFUSE_ERR_INVALID_ARG


def padded(t):
    """Row positions of a split launch: t rounded up to a multiple of 8."""
    return (t + 7) // 8 * 8


@pytest.mark.parametrize("t,d,split,block,grid", [(8, 8192, 4, 256, 32), (8, 8192, 2, 512, 16),
                                                 (1, 4096, 8, 64, 64), (64, 8192, 4, 256, 256),
                                                 (5, 8192, 4, 256, 32), (31, 4096, 8, 64, 256)])
def test_query_launch_split(t, d, split, block, grid):
    """A split launch runs split x (t rounded up to 8) workgroups, a slot each
    (the padding row positions exit at once)."""
    info = arf.arfuse_query_launch(8, t, d, split=split)
    assert (info.grid, info.block, info.vpt, info.split) == (grid, block, 1, split)
    assert info.workspace_bytes == 256 * padded(t)     # two 128-byte lines per row position
    plain = arf.arfuse_query_launch(8, t, d)
    assert (plain.split, plain.workspace_bytes, plain.grid) == (1, 0, t)


# The automatic split for a shape (host-only rule): (n, t, d, layout) -> split
AUTO = [((8, 8, 8192, 0), 8), ((4, 1, 8192, 0), 4), ((8, 64, 8192, 0), 4), ((8, 128, 8192, 0), 2),
        ((8, 129, 8192, 0), 1), ((8, 4096, 8192, 0), 1), ((8, 8, 4096, 0), 1), ((2, 1, 4096, 0), 1),
        ((8, 8, 16384, 0), 8), ((8, 8, 6144, 0), 1), ((8, 8, 8192, 1), 8), ((8, 8, 4096, 1), 8),
        ((4, 8, 4096, 1), 1), ((8, 8, 2048, 1), 1), ((8, 8, 16384, 1), 8), ((8, 32, 65536, 2), 8),
        ((8, 33, 65536, 2), 4), ((8, 65, 65536, 0), 1), ((1, 1, 16, 0), 1), ((8, 8, 8208, 0), 1)]


@pytest.mark.parametrize("shape,split", AUTO)
def test_auto_split_choice(shape, split):
    n, t, d, layout = shape
    info = arf.arfuse_query_launch(n, t, d, layout=layout, split=arf.ARFUSE_SPLIT_AUTO)
    assert info.split == split
    assert info.workspace_bytes == (256 * padded(t) if split > 1 else 0)
    assert info.grid == (padded(t) * split if split > 1 else t)
    assert info.grid <= arf.ARFUSE_MAX_SPLIT_BLOCKS or split == 1
    # the choice is what the explicit split would launch
    if split > 1:
        ex = arf.arfuse_query_launch(n, t, d, layout=layout, split=split)
        assert (ex.grid, ex.block, ex.vpt) == (info.grid, info.block, info.vpt)


def test_auto_split_needs_the_workspace_it_chose():
    o = arf._opts(split=arf.ARFUSE_SPLIT_AUTO)
    assert call(**good(opts=o, d=8192, t=0)) == arf.ARFUSE_OK
    # t = 8, d = 8192 splits 4 ways: without a workspace the call is refused
    assert call(**good(opts=o, d=8192)) == arf.ARFUSE_ERR_INVALID_ARG


def test_status_word_validated():
    """The status word takes device atomics: it must be 8-byte aligned and
    must not share memory with the partials or an output."""
    o = arf._opts(status=spaced(30) + 4)
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(status=spaced(0) + 64)          # inside partial 0
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(status=spaced(10) + 16)         # inside out
    assert call(**good(opts=o)) == arf.ARFUSE_ERR_INVALID_ARG
    o = arf._opts(status=spaced(30))
    assert call(**good(opts=o, t=0)) == arf.ARFUSE_OK


# the all-reduce alone has no exchange: it splits whenever the row reads 32 KiB
AUTO_NO_NORM = [((8, 8, 8192, 0), 8), ((8, 8, 4096, 0), 4), ((4, 8, 8192, 0), 4),
                ((2, 1, 4096, 0), 1), ((8, 64, 8192, 0), 4), ((8, 8, 4096, 1), 8)]


@pytest.mark.parametrize("shape,split", AUTO_NO_NORM)
def test_auto_split_choice_without_norm(shape, split):
    n, t, d, layout = shape
    info = arf.arfuse_query_launch(n, t, d, 0, layout=layout, split=arf.ARFUSE_SPLIT_AUTO)
    assert info.split == split


def test_query_launch_reports_streaming_stores():
    """Calls whose rows take three or more rounds of workgroups (t * vpt >=
    1536) write their outputs through to memory; smaller calls, split rows and
    LL calls keep the other instances."""
    q = arf.arfuse_query_launch
    assert q(8, 4096, 8192).stream_stores == 1
    assert q(8, 1536, 8192).stream_stores == 1
    assert q(8, 1535, 8192).stream_stores == 0
    assert q(8, 1024, 8192).stream_stores == 0
    assert q(8, 512, 8192).stream_stores == 0
    assert q(2, 384, 32768).stream_stores == 1          # vpt 4
    assert q(2, 256, 32768).stream_stores == 0
    assert q(8, 192, 65536).stream_stores == 1          # vpt 8
    assert q(8, 128, 65536).stream_stores == 0
    assert q(8, 4096, 8192, layout=arf.ARFUSE_LAYOUT_LL).stream_stores == 0
    assert q(8, 4096, 8192, layout=arf.ARFUSE_LAYOUT_SENTINEL).stream_stores == 1
    assert q(8, 8, 8192, split=4).stream_stores == 0
    assert q(8, 0, 8192).stream_stores == 0


def test_noalloc_refuses_a_workspace():
    """The allocation-free entry keeps the split exchange in the library's
    own static slots: a caller workspace is an argument error, returned
    before anything else happens (no device lookup, nothing enqueued)."""
    ws = spaced(40)
    o = arf._opts(split=4, workspace=ws, status=spaced(30))
    parts = [spaced(i) for i in range(4)]
    arr = (ctypes.c_void_p * 4)(*parts)
    for t in (0, T):
        rc = arf.lib.arfuse_rmsnorm_noalloc(arr, 4, spaced(8), spaced(9), 1e-5, spaced(10),
                                            spaced(11), None, None, t, 8192, None, ctypes.byref(o))
        assert rc == arf.ARFUSE_ERR_INVALID_ARG
    # the largest split call: 128 row positions (2 slices of 128 rows), 256 bytes each
    assert arf.ARFUSE_NOALLOC_BYTES == arf.ARFUSE_MAX_SPLIT_BLOCKS // 2 * 256 == 32768
    assert max(arf.arfuse_query_launch(8, t, 8192, split=s).workspace_bytes
               for s in (2, 4, 8) for t in range(1, 256 // s + 1)) == arf.ARFUSE_NOALLOC_BYTES
