"""Seeded synthetic inputs for the fused all-reduce epilogue (sum of rank
partials + residual add + RMSNorm, optional FP4 output).

This module is the only code that both the CPU oracle (``oracle/``) and the
HIP path (``reduce_residual_rmsnorm_amd/``) consume. It draws random numbers
and lays them out; it performs none of the method's arithmetic. Conversion of
the drawn float32 values to bfloat16 storage is delegated to PyTorch's CPU
``Tensor.to(torch.bfloat16)`` (round to nearest even), so no rounding code of
this repository is shared between the two sides.

Workload recipe (the pages give the shapes, the distributions are the
synthetic stand-in for real activations):

* ``n`` rank partials, each bf16 ``[t][d]`` row-major, drawn as
  float32 z ~ N(0, 1), scaled in float32 by ``1/sqrt(n)``, stored as bf16.
  They stand in for the row-parallel partial products Z_i whose sum the
  all-reduce forms ("Optimizing Tensor Parallelism Communication Overhead ...",
  "The Anatomy of the Tensor Parallelism Bottleneck").
* residual bf16 ``[t][d]`` ~ N(0, 1); optionally ``round(outlier_frac * t)``
  rows (chosen by the generator, without replacement) are multiplied by 100 in
  float32 before the bf16 store, to stress the row RMS range.
* gamma float32 ``[d]`` ~ U(0.5, 1.5).
* eps = 1e-5 (float32).
* LL flag base: the first uint64 drawn after the data (63-bit range).

Draw order for one call: partials (all ranks, rank-major), residual, gamma,
outlier rows, LL base. ``numpy.random.default_rng(seed)`` is the generator.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

EPS = np.float32(1e-5)

# Byte layout of one LL ("low latency") word: 16 bytes, the first 8 hold four
# bf16 payload elements (element 4w first, little endian), the last 8 hold the
# uint64 flag (little endian). This is the producer-side layout a peer would
# push; the consumer (oracle or kernel) checks the flag and unpacks.
LL_WORD_BYTES = 16
LL_ELEMS_PER_WORD = 4


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via PyTorch's CPU conversion."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    tb = torch.from_numpy(x).to(torch.bfloat16)
    return tb.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening, via PyTorch)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    return tb.to(torch.float32).numpy()


@dataclass
class CallInputs:
    """Inputs of one fused call, host side."""

    n: int
    t: int
    d: int
    partials: np.ndarray          # uint16 [n][t][d] (bf16 bits)
    residual: np.ndarray          # uint16 [t][d]
    gamma: np.ndarray             # float32 [d]
    eps: np.float32
    outlier_rows: np.ndarray      # int64 [k]
    ll_base: int                  # uint64 flag base
    seed: int = 0
    meta: dict = field(default_factory=dict)


def n_outlier_rows(t: int, frac: float) -> int:
    """round(frac * t), Python rounding (half to even)."""
    return int(round(frac * t))


def make_call(n: int, t: int, d: int, seed: int = 0, outlier_frac: float = 0.0,
              gamma_range=(0.5, 1.5)) -> CallInputs:
    """Draw the inputs of one call with the recipe in the module docstring."""
    if n < 1 or t < 0 or d < 0:
        raise ValueError("bad shape")
    rng = np.random.default_rng(seed)
    inv_sqrt_n = np.float32(1.0 / math.sqrt(n))
    parts = np.empty((n, t, d), dtype=np.uint16)
    for i in range(n):
        z = rng.standard_normal((t, d), dtype=np.float32)
        z *= inv_sqrt_n
        parts[i] = to_bf16_bits(z)
    r = rng.standard_normal((t, d), dtype=np.float32)
    g = rng.uniform(gamma_range[0], gamma_range[1], size=d).astype(np.float32)
    k = n_outlier_rows(t, outlier_frac)
    rows = np.sort(rng.choice(t, size=k, replace=False)) if k > 0 else np.zeros(0, np.int64)
    if k > 0:
        r[rows] *= np.float32(100.0)
    res = to_bf16_bits(r)
    base = int(rng.integers(0, 2 ** 63, dtype=np.uint64))
    return CallInputs(n=n, t=t, d=d, partials=parts, residual=res, gamma=g,
                      eps=EPS, outlier_rows=rows.astype(np.int64), ll_base=base,
                      seed=seed)


def make_partial_sets(n: int, t: int, d: int, k: int, seed: int) -> np.ndarray:
    """``k`` independent partial sets, uint16 [k][n][t][d], one per chained call.

    Drawn from ``default_rng(seed)`` with the same per-rank scaling as
    :func:`make_call`."""
    rng = np.random.default_rng(seed)
    inv_sqrt_n = np.float32(1.0 / math.sqrt(n))
    out = np.empty((k, n, t, d), dtype=np.uint16)
    for c in range(k):
        for i in range(n):
            z = rng.standard_normal((t, d), dtype=np.float32)
            z *= inv_sqrt_n
            out[c, i] = to_bf16_bits(z)
    return out


def ll_pack(part: np.ndarray, flag: int) -> np.ndarray:
    """Pack one bf16 [t][d] partial into LL words, uint8 [t][d/4][16].

    ``d`` must be a multiple of 4. Every word carries the same ``flag``."""
    part = np.ascontiguousarray(part, dtype=np.uint16)
    t, d = part.shape
    if d % LL_ELEMS_PER_WORD:
        raise ValueError("d must be a multiple of 4 for LL packing")
    w = d // LL_ELEMS_PER_WORD
    words = np.empty((t, w, 2), dtype=np.uint64)
    payload = part.reshape(t, w, LL_ELEMS_PER_WORD).copy().view(np.uint64).reshape(t, w)
    words[:, :, 0] = payload
    words[:, :, 1] = np.uint64(flag)
    return words.view(np.uint8).reshape(t, w, LL_WORD_BYTES)


def ll_pack_all(parts: np.ndarray, flag: int) -> np.ndarray:
    """LL-pack every rank of uint16 [n][t][d] -> uint8 [n][t][d/4][16]."""
    return np.stack([ll_pack(p, flag) for p in parts])


def ll_set_flag(words: np.ndarray, index, flag: int) -> None:
    """Overwrite the flag of LL word(s) ``index`` of a uint8 [..][16] array in
    place (used to stage stale or corrupted words on the host)."""
    flat = words.reshape(-1, LL_WORD_BYTES)
    view = flat.view(np.uint64).reshape(-1, 2)
    view[index, 1] = np.uint64(flag)


# Named workloads: the shapes the fused call is exercised and measured at.
WORKLOADS = {
    # single decode token, two ranks
    "decode_n2_t1_d4096": dict(n=2, t=1, d=4096, outlier_frac=0.0),
    # Llama-3-8B-shaped decode step (8 ranks, batch 8, hidden 4096), 64 chained calls
    "decode_n8_t8_d4096_chain64": dict(n=8, t=8, d=4096, outlier_frac=0.0, chain=64),
    # Llama-3.1-70B-shaped decode step (hidden 8192, batch 8), 160 chained calls
    "decode_n4_t8_d8192_chain160": dict(n=4, t=8, d=8192, outlier_frac=0.0, chain=160),
    "decode_n8_t8_d8192_chain160": dict(n=8, t=8, d=8192, outlier_frac=0.0, chain=160),
    # prefill bandwidth regime
    "prefill_n8_t512_d8192": dict(n=8, t=512, d=8192, outlier_frac=0.001),
    "prefill_n8_t4096_d8192": dict(n=8, t=4096, d=8192, outlier_frac=0.001),
    # FP4 output
    "fp4_n4_t1_d8192": dict(n=4, t=1, d=8192, outlier_frac=0.001),
    "fp4_n4_t8_d8192": dict(n=4, t=8, d=8192, outlier_frac=0.001),
    "fp4_n4_t64_d8192": dict(n=4, t=64, d=8192, outlier_frac=0.001),
    "fp4_n4_t512_d8192": dict(n=4, t=512, d=8192, outlier_frac=0.001),
}


def make_workload(name: str, seed: int = 0) -> CallInputs:
    w = WORKLOADS[name]
    ci = make_call(w["n"], w["t"], w["d"], seed=seed, outlier_frac=w["outlier_frac"])
    ci.meta = dict(w, name=name)
    return ci
