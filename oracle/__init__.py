"""CPU oracle for the fused all-reduce epilogue + residual + RMSNorm (+ FP4).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this package. The GPU library never imports, links or calls it, and this
package never imports the GPU library.

The arithmetic lives in ``arfuse_oracle.c`` (plain scalar C99, built without
fast-math or FP contraction); this module only builds it with gcc and
marshals numpy arrays through ctypes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "arfuse_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True, out: Optional[str] = None, extra_flags: Sequence[str] = (),
          src: Optional[str] = None) -> str:
    """Compile the oracle into a shared library with gcc and return its path."""
    out = out or _LIB
    src = src or _SRC
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    c = ctypes
    P = c.c_void_p
    I64 = c.c_int64
    lib.oracle_bf16_to_f32.argtypes = [c.c_uint16]
    lib.oracle_bf16_to_f32.restype = c.c_float
    lib.oracle_bf16_rne.argtypes = [c.c_float]
    lib.oracle_bf16_rne.restype = c.c_uint16
    lib.oracle_bf16_rne_array.argtypes = [P, I64, P]
    lib.oracle_e4m3_value.argtypes = [c.c_uint8]
    lib.oracle_e4m3_value.restype = c.c_double
    lib.oracle_e4m3_rne.argtypes = [c.c_float]
    lib.oracle_e4m3_rne.restype = c.c_uint8
    lib.oracle_e4m3_rne_array.argtypes = [P, I64, P]
    lib.oracle_e2m1_value.argtypes = [c.c_uint8]
    lib.oracle_e2m1_value.restype = c.c_double
    lib.oracle_e2m1_rne.argtypes = [c.c_float]
    lib.oracle_e2m1_rne.restype = c.c_uint8
    lib.oracle_e2m1_rne_array.argtypes = [P, I64, P]
    lib.oracle_quantize_fp4.argtypes = [P, I64, I64, P, P]
    lib.oracle_allreduce_rmsnorm.argtypes = [P, c.c_int, P, P, c.c_float, I64, I64,
                                             P, P, P, P, P]
    lib.oracle_allreduce_rmsnorm.restype = c.c_int
    lib.oracle_rank_sum_residual.argtypes = [P, c.c_int, P, I64, I64, P]
    lib.oracle_rank_sum_residual.restype = c.c_int
    lib.oracle_rmsnorm_rows.argtypes = [P, P, c.c_float, I64, I64, P]
    lib.oracle_rmsnorm_rows.restype = c.c_int
    lib.oracle_ll_unpack.argtypes = [P, I64, c.c_uint64, P]
    lib.oracle_ll_unpack.restype = c.c_int64
    lib.oracle_quantize_fp8.argtypes = [P, I64, I64, c.c_float, P]
    lib.oracle_fused.argtypes = [P, c.c_int, P, P, c.c_float, I64, I64, P, P, P, P, P, P, c.c_float]
    lib.oracle_fused.restype = c.c_int
    lib.oracle_sentinel_pending.argtypes = [P, I64, c.c_uint16]
    lib.oracle_sentinel_pending.restype = c.c_int64
    return lib


def load(path: Optional[str] = None):
    """Load the oracle library (building it first only if it is missing)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """Array-level wrapper over one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # ---- scalar format helpers (vectorised over numpy arrays)
    def bf16_rne(self, x) -> np.ndarray:
        x = _c(x, np.float32)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_bf16_rne_array(_ptr(x), x.size, _ptr(out))
        return out

    def e4m3_rne(self, x) -> np.ndarray:
        x = _c(x, np.float32)
        out = np.empty(x.shape, np.uint8)
        self.lib.oracle_e4m3_rne_array(_ptr(x), x.size, _ptr(out))
        return out

    def e4m3_value(self, code: int) -> float:
        return self.lib.oracle_e4m3_value(int(code))

    def e2m1_rne(self, q) -> np.ndarray:
        q = _c(q, np.float32)
        out = np.empty(q.shape, np.uint8)
        self.lib.oracle_e2m1_rne_array(_ptr(q), q.size, _ptr(out))
        return out

    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(int(code))

    # ---- method steps
    def quantize_fp4(self, y):
        y = _c(y, np.float32)
        t, d = y.shape
        codes = np.empty((t, d // 2), np.uint8)
        scales = np.empty((t, d // 16), np.uint8)
        self.lib.oracle_quantize_fp4(_ptr(y), t, d, _ptr(codes), _ptr(scales))
        return codes, scales

    def rank_sum_residual(self, partials, residual) -> np.ndarray:
        parts = [_c(p, np.uint16) for p in partials]
        res = _c(residual, np.uint16)
        t, d = res.shape
        arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
        h = np.empty((t, d), np.float32)
        rc = self.lib.oracle_rank_sum_residual(arr, len(parts), _ptr(res), t, d, _ptr(h))
        if rc != 0:
            raise ValueError("oracle_rank_sum_residual rejected its arguments")
        return h

    def rmsnorm_rows(self, h, gamma, eps) -> np.ndarray:
        h = _c(h, np.float32)
        g = _c(gamma, np.float32)
        t, d = h.shape
        y = np.empty((t, d), np.float32)
        rc = self.lib.oracle_rmsnorm_rows(_ptr(h), _ptr(g), float(eps), t, d, _ptr(y))
        if rc != 0:
            raise ValueError("oracle_rmsnorm_rows rejected its arguments")
        return y

    def allreduce_rmsnorm(self, partials, residual, gamma, eps, fp4: bool = False,
                          want_out: bool = True):
        """Run the fused call. Returns dict(residual_out, y32, out, codes, scales)."""
        parts = [_c(p, np.uint16) for p in partials]
        res = _c(residual, np.uint16)
        g = _c(gamma, np.float32)
        t, d = res.shape
        arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
        r_out = np.empty((t, d), np.uint16)
        y32 = np.empty((t, d), np.float32)
        out = np.empty((t, d), np.uint16) if want_out else None
        codes = np.empty((t, d // 2), np.uint8) if fp4 else None
        scales = np.empty((t, d // 16), np.uint8) if fp4 else None
        nul = ctypes.c_void_p(0)
        rc = self.lib.oracle_allreduce_rmsnorm(
            arr, len(parts), _ptr(res), _ptr(g), float(eps), t, d, _ptr(r_out), _ptr(y32),
            _ptr(out) if out is not None else nul,
            _ptr(codes) if fp4 else nul, _ptr(scales) if fp4 else nul)
        if rc != 0:
            raise ValueError("oracle_allreduce_rmsnorm rejected its arguments")
        return dict(residual_out=r_out, y32=y32, out=out, codes=codes, scales=scales)

    def quantize_fp8(self, y, inv_scale):
        y = _c(y, np.float32)
        out = np.empty(y.shape, np.uint8)
        t, d = y.shape
        self.lib.oracle_quantize_fp8(_ptr(y), t, d, float(inv_scale), _ptr(out))
        return out

    def fused(self, partials, residual, gamma, eps, t=None, d=None, out=True, fp4=False,
              fp8_inv_scale=None, residual_out=True):
        """Any pattern: residual and/or gamma may be None. Returns a dict."""
        parts = [_c(p, np.uint16) for p in partials]
        t, d = parts[0].shape if t is None else (t, d)
        res = _c(residual, np.uint16) if residual is not None else None
        g = _c(gamma, np.float32) if gamma is not None else None
        arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
        nul = ctypes.c_void_p(0)
        norm = g is not None
        r = dict(residual_out=np.empty((t, d), np.uint16) if residual_out else None,
                 y32=np.empty((t, d), np.float32) if norm else None,
                 out=np.empty((t, d), np.uint16) if (norm and out) else None,
                 codes=np.empty((t, d // 2), np.uint8) if (norm and fp4) else None,
                 scales=np.empty((t, d // 16), np.uint8) if (norm and fp4) else None,
                 fp8=np.empty((t, d), np.uint8) if (norm and fp8_inv_scale is not None) else None)
        pp = {k: (_ptr(v) if v is not None else nul) for k, v in r.items()}
        rc = self.lib.oracle_fused(arr, len(parts), _ptr(res) if res is not None else nul,
                                   _ptr(g) if g is not None else nul, float(eps), t, d,
                                   pp["residual_out"], pp["y32"], pp["out"], pp["codes"],
                                   pp["scales"], pp["fp8"],
                                   float(fp8_inv_scale if fp8_inv_scale is not None else 1.0))
        if rc != 0:
            raise ValueError("oracle_fused rejected its arguments")
        return r

    def sentinel_pending(self, part, sentinel: int) -> int:
        p = _c(part, np.uint16)
        n = self.lib.oracle_sentinel_pending(_ptr(p), p.size, int(sentinel))
        if n < 0:
            raise ValueError("oracle_sentinel_pending rejected its arguments")
        return int(n)

    def ll_unpack(self, words, n_elems: int, flag: int):
        w = _c(words, np.uint8)
        out = np.empty(n_elems, np.uint16)
        bad = self.lib.oracle_ll_unpack(_ptr(w), n_elems, ctypes.c_uint64(flag), _ptr(out))
        if bad < 0:
            raise ValueError("oracle_ll_unpack rejected its arguments")
        return out, int(bad)

    def chain(self, partial_sets, residual0, gamma, eps, k: int, fp4: bool = False,
              per_call: bool = False):
        """Replay ``k`` chained calls: call c consumes call c-1's residual_out
        (Deep Dive: AllReduce and AllReduce Fusion in TensorRT-LLM, §6.2:
        each layer's fused call takes the residual the previous one wrote).

        ``per_call=False``: ``partial_sets`` is one sequence of N partials,
        read by every call (the same buffers). ``per_call=True``: it is a
        sequence of exactly k such sequences and call c reads the c-th.
        Returns the list of per-call result dicts."""
        if per_call and len(partial_sets) != k:
            raise ValueError("per_call needs one partial set per call (%d sets, %d calls)"
                             % (len(partial_sets), k))
        res = _c(residual0, np.uint16)
        results = []
        for c in range(k):
            parts = partial_sets[c] if per_call else partial_sets
            r = self.allreduce_rmsnorm(parts, res, gamma, eps, fp4=fp4)
            results.append(r)
            res = r["residual_out"]
        return results


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
