"""Helpers of the GPU tests: move seeded inputs to the device, run the fused
call through the C ABI binding, and compare with the oracle to the
acceptance bar (residual_out bit-exact; bf16 y within 1.6e-2 + 8e-3 |y32|
of the oracle's fp32 y; FP4 codes at most one E2M1 step off on at most 1e-4
of elements, scales likewise)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si

DEV = "cuda:0"
Y_ATOL = 1.6e-2
Y_RTOL = 8e-3
FP4_MISMATCH_FRAC = 1e-4


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case] %s" % msg, flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (host) -> bf16 tensor on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_u16(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_empty(t, d):
    return torch.empty((t, d), dtype=torch.bfloat16, device=DEV)


class Dev:
    """Device copies of one call's inputs plus output buffers."""

    def __init__(self, ci: si.CallInputs, fp4=False, out=True, ll_flag=None):
        t, d = ci.t, ci.d
        self.ci = ci
        if ll_flag is None:
            self.parts = [dev_u16(p) for p in ci.partials]
        else:
            self.parts = [dev_u8(si.ll_pack(p, ll_flag)) for p in ci.partials]
        self.residual = dev_u16(ci.residual)
        self.gamma = dev_f32(ci.gamma)
        self.out = bf16_empty(t, d) if out else None
        self.residual_out = bf16_empty(t, d)
        self.codes = torch.empty((t, d // 2), dtype=torch.uint8, device=DEV) if fp4 else None
        self.scales = torch.empty((t, d // 16), dtype=torch.uint8, device=DEV) if fp4 else None

    def run(self, eps=None, **opts):
        ci = self.ci
        eps = ci.eps if eps is None else eps
        if opts:
            arf.arfuse_rmsnorm_ex(self.parts, self.residual, self.gamma, eps, self.out,
                                  self.residual_out, self.codes, self.scales, t=ci.t, d=ci.d,
                                  **opts)
        else:
            arf.arfuse_rmsnorm(self.parts, self.residual, self.gamma, eps, self.out,
                               self.residual_out, self.codes, self.scales, t=ci.t, d=ci.d)
        return self

    def fetch(self):
        torch.cuda.synchronize()
        r = dict(residual_out=host_u16(self.residual_out))
        r["out"] = host_u16(self.out) if self.out is not None else None
        r["codes"] = self.codes.cpu().numpy() if self.codes is not None else None
        r["scales"] = self.scales.cpu().numpy() if self.scales is not None else None
        return r


# ------------------------------------------------------------- comparisons

def assert_residual_exact(got: np.ndarray, want: np.ndarray, what="residual_out"):
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, "%s: %d of %d elements differ, first at %s (0x%04x vs 0x%04x)" % (
        what, bad.size, got.size, np.unravel_index(bad[0], got.shape), got.reshape(-1)[bad[0]],
        want.reshape(-1)[bad[0]])


def y_errors(out_bits: np.ndarray, y32: np.ndarray):
    g = si.bf16_bits_to_f32(out_bits).astype(np.float64)
    y = y32.astype(np.float64)
    err = np.abs(g - y)
    rel = err / np.maximum(np.abs(y), 1e-30)
    return err, rel


def assert_y_close(out_bits: np.ndarray, y32: np.ndarray, want_bits: np.ndarray = None):
    err, rel = y_errors(out_bits, y32)
    bound = Y_ATOL + Y_RTOL * np.abs(y32.astype(np.float64))
    bad = np.nonzero((err > bound).reshape(-1))[0]
    assert bad.size == 0, "y: %d elements outside %.3g + %.3g|y| (max abs err %.3g)" % (
        bad.size, Y_ATOL, Y_RTOL, err.max())
    stats = dict(max_abs=float(err.max()), max_rel=float(rel[np.abs(y32) > 1e-3].max())
                 if (np.abs(y32) > 1e-3).any() else 0.0)
    if want_bits is not None:
        stats["bf16_equal_frac"] = float((out_bits == want_bits).mean())
    return stats


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    t, h = codes.shape
    c = np.empty((t, 2 * h), np.uint8)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    return c


def assert_fp4_close(codes, scales, want_codes, want_scales, frac=FP4_MISMATCH_FRAC):
    """End-to-end FP4 bar: at most `frac` of codes differ, each by one E2M1
    step with the same sign; scales likewise at most `frac` of blocks, one
    E4M3 step."""
    g, w = unpack_codes(codes).astype(np.int16), unpack_codes(want_codes).astype(np.int16)
    diff = g != w
    n_bad = int(diff.sum())
    if n_bad:
        gs, ws = g[diff] >> 3, w[diff] >> 3
        gm, wm = g[diff] & 7, w[diff] & 7
        assert np.all(gs == ws), "FP4 sign differs"
        assert np.abs(gm - wm).max() <= 1, "FP4 code off by more than one step"
    assert n_bad <= frac * g.size, "FP4: %d of %d codes differ" % (n_bad, g.size)
    sd = scales.astype(np.int16) != want_scales.astype(np.int16)
    if sd.any():
        assert np.abs(scales.astype(np.int16) - want_scales.astype(np.int16)).max() <= 1
    assert sd.sum() <= frac * scales.size, "FP4: %d of %d scales differ" % (sd.sum(), scales.size)
    return dict(code_mismatch=n_bad, scale_mismatch=int(sd.sum()))
