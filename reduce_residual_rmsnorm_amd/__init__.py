"""Python binding of the arfuse C ABI (include/arfuse.h): argument marshalling
only. Every step of the fused call runs in the gfx950 kernels of
``lib/libarfuse.so``; PyTorch provides device memory and streams.

Build the library first (``python reduce_residual_rmsnorm_amd/build.py`` or
``__graft_entry__.build()``); importing this package without it fails.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libarfuse.so")

ARFUSE_OK = 0
ARFUSE_ERR_INVALID_ARG = 1
ARFUSE_ERR_UNSUPPORTED = 2
ARFUSE_ERR_LAUNCH = 3
ARFUSE_ERR_FLAG_TIMEOUT = 4
ARFUSE_LAYOUT_PLAIN = 0
ARFUSE_LAYOUT_LL = 1
ARFUSE_LAYOUT_SENTINEL = 2
ARFUSE_SENTINEL_DEFAULT = 0xFFFF
ARFUSE_EPI_FP8 = 4
ARFUSE_EPI_BF16 = 1
ARFUSE_EPI_FP4 = 2
ARFUSE_MAX_PARTIALS = 8
ARFUSE_MAX_D = 65536
ARFUSE_MAX_POLLS = 1 << 20
ARFUSE_MAX_SPLIT = 8
ARFUSE_MAX_SPLIT_BLOCKS = 256
ARFUSE_SPLIT_AUTO = 0xFFFFFFFF
ARFUSE_NOALLOC_BYTES = 32768

# The exported functions, as declared in include/arfuse.h.
EXPORTED = ("arfuse_rmsnorm", "arfuse_rmsnorm_ex", "arfuse_rmsnorm_noalloc",
            "arfuse_quantize_fp4", "arfuse_quantize_fp4_ll",
            "arfuse_query_launch", "arfuse_launch_floor", "arfuse_stream_copy", "arfuse_stream_mix",
            "arfuse_round_bf16", "arfuse_round_fp8", "arfuse_round_fp4",
            "arfuse_status_string", "arfuse_version")


class ArfuseError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code & 0xFF
        self.hip_error = code >> 8
        msg = "%s: %s (status %d)" % (where, arfuse_status_string(code), self.code)
        if self.hip_error:
            msg += ", hipError_t %d" % self.hip_error
        super().__init__(msg)


class arfuse_ll_status(ctypes.Structure):
    _fields_ = [("code", ctypes.c_uint32), ("exchange_timeouts", ctypes.c_uint32),
                ("bad_words", ctypes.c_uint64)]


class arfuse_opts(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("max_polls", ctypes.c_uint32),
                ("ll_flag", ctypes.c_uint64), ("status", ctypes.c_void_p),
                ("block_threads", ctypes.c_int32), ("vpt", ctypes.c_int32),
                ("sentinel", ctypes.c_uint32), ("split", ctypes.c_uint32),
                ("reset", ctypes.c_void_p), ("fp8_out", ctypes.c_void_p),
                ("fp8_inv_scale", ctypes.c_float), ("reserved2", ctypes.c_uint32),
                ("workspace", ctypes.c_void_p)]


class arfuse_launch_info(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int64), ("block", ctypes.c_int32), ("vpt", ctypes.c_int32),
                ("split", ctypes.c_int32), ("stream_stores", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


def _load(path: str = LIB_PATH):
    # PyTorch's ROCm wheel carries its own HIP runtime (libamdhip64.so.7) and
    # finds it by path. If libarfuse.so were loaded first it would pull in the
    # system runtime under the same soname and the process would hold two HIP
    # runtimes, each rejecting the other's streams. Importing torch first makes
    # the dynamic linker bind libarfuse.so to the runtime torch already loaded.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError("libarfuse.so is not built (%s); run `python "
                          "reduce_residual_rmsnorm_amd/build.py`" % path)
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    common = [P, I, P, P, ctypes.c_float, P, P, P, P, I64, I64, P]
    lib.arfuse_rmsnorm.argtypes = common
    lib.arfuse_rmsnorm.restype = I
    lib.arfuse_rmsnorm_ex.argtypes = common + [ctypes.POINTER(arfuse_opts)]
    lib.arfuse_rmsnorm_ex.restype = I
    lib.arfuse_rmsnorm_noalloc.argtypes = common + [ctypes.POINTER(arfuse_opts)]
    lib.arfuse_rmsnorm_noalloc.restype = I
    lib.arfuse_quantize_fp4.argtypes = [P, I64, I64, P, P, P]
    lib.arfuse_quantize_fp4.restype = I
    lib.arfuse_quantize_fp4_ll.argtypes = [P, I64, I64, P, P, P]
    lib.arfuse_quantize_fp4_ll.restype = I
    lib.arfuse_stream_mix.argtypes = [P, I, P, I, I64, I64, P]
    lib.arfuse_stream_mix.restype = I
    lib.arfuse_query_launch.argtypes = [I, I64, I64, I, ctypes.POINTER(arfuse_opts),
                                        ctypes.POINTER(arfuse_launch_info)]
    lib.arfuse_query_launch.restype = I
    lib.arfuse_launch_floor.argtypes = [I, I64, I64, I, ctypes.POINTER(arfuse_opts), P]
    lib.arfuse_launch_floor.restype = I
    lib.arfuse_stream_copy.argtypes = [P, P, I64, P]
    lib.arfuse_stream_copy.restype = I
    lib.arfuse_round_bf16.argtypes = [P, I64, P, P]
    lib.arfuse_round_bf16.restype = I
    lib.arfuse_round_fp8.argtypes = [P, I64, P, P]
    lib.arfuse_round_fp8.restype = I
    lib.arfuse_round_fp4.argtypes = [P, I64, P, P]
    lib.arfuse_round_fp4.restype = I
    lib.arfuse_status_string.argtypes = [I]
    lib.arfuse_status_string.restype = ctypes.c_char_p
    lib.arfuse_version.argtypes = []
    lib.arfuse_version.restype = I
    return lib


lib = _load()


# ---------------------------------------------------------------- marshalling

def _addr(x) -> int:
    """Device address of a tensor, or an int address, or 0 for None."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _buf(x, nbytes: int, name: str) -> int:
    """Device address of a buffer argument. A tensor must live on a GPU, be
    contiguous and hold at least `nbytes` bytes (any dtype: bf16 data may come
    as a bfloat16, int16 or uint8 view); an int is taken as a raw device
    address; None is NULL. Checked here because the C ABI receives bare
    pointers: a host tensor's address would make the kernel fault."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("%s must be a GPU tensor (got device %s)" % (name, x.device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes; the call needs %d" % (name, have, nbytes))
    return int(x.data_ptr())


def _call_buffers(partials, residual, gamma, out, residual_out, fp4_out, fp4_scales, t, d,
                  layout=ARFUSE_LAYOUT_PLAIN, fp8_out=None, status=None, reset=None, split=0,
                  workspace=None):
    """Checked addresses of every buffer of a fused call (see _buf)."""
    plane = t * d * 2
    pbytes = 2 * plane if layout == ARFUSE_LAYOUT_LL else plane
    arr = (ctypes.c_void_p * len(partials))(
        *[_buf(p, pbytes, "partials[%d]" % i) for i, p in enumerate(partials)])
    return dict(
        arr=arr,
        residual=_buf(residual, plane, "residual"),
        gamma=_buf(gamma, 4 * d if t else 0, "gamma"),
        out=_buf(out, plane, "out"),
        residual_out=_buf(residual_out, plane, "residual_out"),
        fp4_out=_buf(fp4_out, t * d // 2, "fp4_out"),
        fp4_scales=_buf(fp4_scales, t * d // 16, "fp4_scales"),
        fp8_out=_buf(fp8_out, t * d, "fp8_out"),
        status=_buf(status, 16, "status"),
        # an unsplit call never touches the workspace; a split one uses 256
        # bytes per row position (t rounded up to a multiple of 8)
        workspace=_buf(workspace, 256 * ((t + 7) // 8 * 8) if int(split) > 1 else 0,
                       "workspace"),
        reset=None if reset is None else [_buf(r, plane, "reset[%d]" % i)
                                          for i, r in enumerate(reset)])


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _opts(layout=ARFUSE_LAYOUT_PLAIN, ll_flag=0, max_polls=0, status=None, block_threads=0,
          vpt=0, sentinel=0, reset=None, fp8_out=None, fp8_inv_scale=1.0, split=0,
          workspace=None):
    """Build an arfuse_opts; returns (opts, keepalive) - the host array of
    reset pointers must outlive the call."""
    keep = None
    reset_addr = 0
    if reset is not None:
        keep = (ctypes.c_void_p * len(reset))(*[_addr(r) for r in reset])
        reset_addr = ctypes.addressof(keep)
    o = arfuse_opts(layout=int(layout), max_polls=int(max_polls), ll_flag=int(ll_flag),
                    status=_addr(status), block_threads=int(block_threads), vpt=int(vpt),
                    sentinel=int(sentinel), split=int(split), reset=reset_addr,
                    fp8_out=_addr(fp8_out), fp8_inv_scale=float(fp8_inv_scale), reserved2=0,
                    workspace=_addr(workspace))
    o._keep = keep
    return o


def _check(rc: int, where: str) -> None:
    if rc != ARFUSE_OK:
        raise ArfuseError(rc, where)


def _td(residual, t, d):
    if t is None or d is None:
        t, d = residual.shape
    return int(t), int(d)


# ---------------------------------------------------------------- entry points

def arfuse_rmsnorm(partials: Sequence, residual, gamma, eps: float, out, residual_out,
                   fp4_out=None, fp4_scales=None, stream=None, t=None, d=None) -> None:
    """Fused call on plain bf16 partials; see arfuse_rmsnorm in include/arfuse.h.
    Tensors (or int device addresses with explicit t, d) are passed through."""
    t, d = _td(residual, t, d)
    b = _call_buffers(partials, residual, gamma, out, residual_out, fp4_out, fp4_scales, t, d)
    rc = lib.arfuse_rmsnorm(b["arr"], len(partials), b["residual"], b["gamma"], float(eps),
                            b["out"], b["residual_out"], b["fp4_out"], b["fp4_scales"],
                            t, d, _stream(stream))
    _check(rc, "arfuse_rmsnorm")


def arfuse_rmsnorm_ex(partials: Sequence, residual, gamma, eps: float, out, residual_out,
                      fp4_out=None, fp4_scales=None, stream=None, t=None, d=None, *,
                      layout=ARFUSE_LAYOUT_PLAIN, ll_flag=0, max_polls=0, status=None,
                      block_threads=0, vpt=0, sentinel=0, reset=None, fp8_out=None,
                      fp8_inv_scale=1.0, split=0, workspace=None) -> None:
    """Fused call with options; see arfuse_rmsnorm_ex in include/arfuse.h.
    residual and gamma may be None (the no-residual and all-reduce-only
    patterns); then pass t and d explicitly. split > 1 divides each row
    between that many workgroups, which exchange their sums of squares
    through `workspace` (256 bytes per row position, t rounded up to a
    multiple of 8; never needs clearing);
    ARFUSE_SPLIT_AUTO lets the library choose (arfuse_query_launch tells
    the choice and the workspace size)."""
    t, d = _td(residual, t, d)
    ws_split = int(split)
    if ws_split == ARFUSE_SPLIT_AUTO:   # the workspace the library's choice needs
        info = arfuse_launch_info()
        q = _opts(layout=layout, split=split)
        epi = ((ARFUSE_EPI_BF16 if out is not None else 0) |
               (ARFUSE_EPI_FP4 if fp4_out is not None else 0) |
               (ARFUSE_EPI_FP8 if fp8_out is not None else 0))
        ws_split = (info.split if lib.arfuse_query_launch(len(partials), t, d, epi,
                                                          ctypes.byref(q), ctypes.byref(info)) == 0
                    else 1)
    b = _call_buffers(partials, residual, gamma, out, residual_out, fp4_out, fp4_scales, t, d,
                      layout=layout, fp8_out=fp8_out, status=status, reset=reset, split=ws_split,
                      workspace=workspace)
    o = _opts(layout, ll_flag, max_polls, b["status"], block_threads, vpt, sentinel, b["reset"],
              b["fp8_out"], fp8_inv_scale, split, b["workspace"])
    rc = lib.arfuse_rmsnorm_ex(b["arr"], len(partials), b["residual"], b["gamma"], float(eps),
                               b["out"], b["residual_out"], b["fp4_out"], b["fp4_scales"],
                               t, d, _stream(stream), ctypes.byref(o))
    _check(rc, "arfuse_rmsnorm_ex")


def arfuse_rmsnorm_noalloc(partials: Sequence, residual, gamma, eps: float, out, residual_out,
                           fp4_out=None, fp4_scales=None, stream=None, t=None, d=None, *,
                           layout=ARFUSE_LAYOUT_PLAIN, ll_flag=0, max_polls=0, status=None,
                           block_threads=0, vpt=0, sentinel=0, reset=None, fp8_out=None,
                           fp8_inv_scale=1.0, split=0) -> None:
    """arfuse_rmsnorm_ex without a workspace: split rows exchange through the
    library's static slots (for callers that cannot allocate); see
    arfuse_rmsnorm_noalloc in include/arfuse.h."""
    t, d = _td(residual, t, d)
    b = _call_buffers(partials, residual, gamma, out, residual_out, fp4_out, fp4_scales, t, d,
                      layout=layout, fp8_out=fp8_out, status=status, reset=reset)
    o = _opts(layout, ll_flag, max_polls, b["status"], block_threads, vpt, sentinel, b["reset"],
              b["fp8_out"], fp8_inv_scale, split, None)
    rc = lib.arfuse_rmsnorm_noalloc(b["arr"], len(partials), b["residual"], b["gamma"],
                                    float(eps), b["out"], b["residual_out"], b["fp4_out"],
                                    b["fp4_scales"], t, d, _stream(stream), ctypes.byref(o))
    _check(rc, "arfuse_rmsnorm_noalloc")


def arfuse_quantize_fp4(y, codes, scales, stream=None, t=None, d=None) -> None:
    """FP4 epilogue alone on fp32 y [t][d]; see include/arfuse.h."""
    if t is None or d is None:
        t, d = y.shape
    t, d = int(t), int(d)
    rc = lib.arfuse_quantize_fp4(_buf(y, 4 * t * d, "y"), t, d, _buf(codes, t * d // 2, "codes"),
                                 _buf(scales, t * d // 16, "scales"), _stream(stream))
    _check(rc, "arfuse_quantize_fp4")


def arfuse_quantize_fp4_ll(y, codes, scales, stream=None, t=None, d=None) -> None:
    """Test entry: the LL-layout FP4 epilogue alone on fp32 y [t][d]; see
    include/arfuse.h."""
    if t is None or d is None:
        t, d = y.shape
    t, d = int(t), int(d)
    rc = lib.arfuse_quantize_fp4_ll(_buf(y, 4 * t * d, "y"), t, d,
                                    _buf(codes, t * d // 2, "codes"),
                                    _buf(scales, t * d // 16, "scales"), _stream(stream))
    _check(rc, "arfuse_quantize_fp4_ll")


def arfuse_stream_mix(inputs: Sequence, outputs: Sequence, t: int, d: int, stream=None) -> None:
    """Measurement aid: the fused call's byte mix in its launch shape; see
    include/arfuse.h."""
    t, d = int(t), int(d)
    plane = t * d * 2
    ia = (ctypes.c_void_p * len(inputs))(*[_buf(x, plane, "inputs[%d]" % i)
                                           for i, x in enumerate(inputs)])
    oa = (ctypes.c_void_p * len(outputs))(*[_buf(x, plane, "outputs[%d]" % i)
                                            for i, x in enumerate(outputs)])
    rc = lib.arfuse_stream_mix(ia, len(inputs), oa, len(outputs), t, d, _stream(stream))
    _check(rc, "arfuse_stream_mix")


def arfuse_query_launch(n_partials: int, t: int, d: int, epilogue: int = ARFUSE_EPI_BF16,
                        **opts) -> arfuse_launch_info:
    info = arfuse_launch_info()
    o = _opts(**opts)
    rc = lib.arfuse_query_launch(int(n_partials), int(t), int(d), int(epilogue),
                                 ctypes.byref(o), ctypes.byref(info))
    _check(rc, "arfuse_query_launch")
    return info


def arfuse_launch_floor(n_partials: int, t: int, d: int, epilogue: int = ARFUSE_EPI_BF16,
                        stream=None, **opts) -> None:
    o = _opts(**opts)
    rc = lib.arfuse_launch_floor(int(n_partials), int(t), int(d), int(epilogue),
                                 ctypes.byref(o), _stream(stream))
    _check(rc, "arfuse_launch_floor")


def arfuse_stream_copy(dst, src, nbytes: Optional[int] = None, stream=None) -> None:
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    nbytes = int(nbytes)
    rc = lib.arfuse_stream_copy(_buf(dst, nbytes, "dst"), _buf(src, nbytes, "src"), nbytes,
                                _stream(stream))
    _check(rc, "arfuse_stream_copy")


def arfuse_round_bf16(x, out, stream=None) -> None:
    """Test entry: the kernel's fp32 -> bf16 rounding of x into out."""
    n = int(x.numel())
    rc = lib.arfuse_round_bf16(_buf(x, 4 * n, "x"), n, _buf(out, 2 * n, "out"), _stream(stream))
    _check(rc, "arfuse_round_bf16")


def arfuse_round_fp8(x, out, stream=None) -> None:
    """Test entry: the kernel's FP8 conversion (inv_scale 1) of x into out."""
    n = int(x.numel())
    rc = lib.arfuse_round_fp8(_buf(x, 4 * n, "x"), n, _buf(out, n, "out"), _stream(stream))
    _check(rc, "arfuse_round_fp8")


def arfuse_round_fp4(x, out, stream=None) -> None:
    """Test entry: the FP4 conversion of the kernel's fast FP4 path (scale 1)
    of x (fp32, n even) into out (n / 2 bytes)."""
    n = int(x.numel())
    rc = lib.arfuse_round_fp4(_buf(x, 4 * n, "x"), n, _buf(out, n // 2, "out"), _stream(stream))
    _check(rc, "arfuse_round_fp4")


def arfuse_status_string(code: int) -> str:
    return lib.arfuse_status_string(int(code)).decode()


def arfuse_version() -> int:
    return lib.arfuse_version()
