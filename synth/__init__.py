"""Seeded synthetic workloads for the Muon optimizer step.

This module only draws inputs.  It holds none of the optimizer's arithmetic
(no momentum, no normalisation, no Newton-Schulz, no update), so both the
CPU oracle and the GPU path can consume what it produces without sharing any
of the method's code.

Gradient recipe (low rank plus noise, the "nearly low-rank, badly
conditioned" updates that the Muon synthesis note on
papers.chlience.com describes in its section 6):

    G = (1/4) * P @ Q + sigma * N,   P: rows x k,  Q: k x cols,  N: rows x cols

with every entry of P, Q and N iid N(0, 1).  Initial weights are
W0 = 0.02 * N(0, 1), initial momentum B0 = 0.

Two generators exist:

* ``numpy_matrix``: float64 draws from ``numpy.random.default_rng`` seeded
  with ``[workload_id, matrix_index, step, tag]`` (tag 0 = gradient,
  tag 1 = initial weights), drawn in the order P, Q, N, then rounded to
  float32 with round-to-nearest-even (and, for bf16 gradients, from that
  float32 to bf16, again round-to-nearest-even).  Used for every case small
  enough for the CPU.
* ``torch_matrix``: the same recipe drawn with a seeded ``torch.Generator``
  on a device (float32 draws).  Used where the full-size workloads are too
  large to draw on the host in reasonable time; sampled matrices are copied
  back to the host and handed to the oracle as they are.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    name: str


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int               # seed component
    name: str
    matrices: Tuple[MatrixSpec, ...]
    rank: int              # k of the low-rank part
    noise: float           # sigma of the noise part
    g_dtype: str           # "f32" or "bf16"
    steps: int             # consecutive optimizer steps the case runs
    mu: float = 0.95
    lr: float = 0.02
    scale: float = 1.0

    @property
    def n_params(self) -> int:
        return sum(m.rows * m.cols for m in self.matrices)


def _layers(n_layers: int, d: int, d_ff: int) -> Tuple[MatrixSpec, ...]:
    out: List[MatrixSpec] = []
    for layer in range(n_layers):
        for nm in ("q", "k", "v", "o"):
            out.append(MatrixSpec(d, d, f"l{layer}.{nm}"))
        out.append(MatrixSpec(d, d_ff, f"l{layer}.fc"))
        out.append(MatrixSpec(d_ff, d, f"l{layer}.proj"))
    return tuple(out)


def _moe_share() -> Tuple[MatrixSpec, ...]:
    out: List[MatrixSpec] = []
    out += [MatrixSpec(2048, 7168, f"expert{i}.up") for i in range(64)]
    out += [MatrixSpec(7168, 2048, f"expert{i}.down") for i in range(64)]
    out += [MatrixSpec(4096, 14336, f"dense{i}") for i in range(8)]
    return tuple(out)


WORKLOADS = {
    "single256": Workload(0, "single256", (MatrixSpec(256, 256, "w"),), 16, 0.1, "f32", 1),
    "gpt2s_fc_10step": Workload(1, "gpt2s_fc_10step", (MatrixSpec(768, 3072, "fc"),), 16, 0.1, "f32", 10),
    "gpt2_small": Workload(2, "gpt2_small", _layers(12, 768, 3072), 16, 0.1, "f32", 1),
    "gpt2_xl_1p5b": Workload(3, "gpt2_xl_1p5b", _layers(48, 1600, 6400), 32, 0.1, "f32", 1),
    "moe_share": Workload(4, "moe_share", _moe_share(), 64, 0.05, "bf16", 1),
}
ORDER = ("single256", "gpt2s_fc_10step", "gpt2_small", "gpt2_xl_1p5b", "moe_share")


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- numpy side
def _rng(wid: int, idx: int, step: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([wid, idx, step, tag])


def numpy_gradient(rows: int, cols: int, rank: int, noise: float, g_dtype: str,
                   seed: Sequence[int]) -> np.ndarray:
    """One gradient.  Returns float32, or uint16 bf16 bits when g_dtype == 'bf16'."""
    rng = np.random.default_rng(list(seed))
    p = rng.standard_normal((rows, rank))
    q = rng.standard_normal((rank, cols))
    n = rng.standard_normal((rows, cols))
    g = (0.25 * (p @ q) + noise * n).astype(np.float32)
    if g_dtype == "bf16":
        return f32_to_bf16_bits(g)
    if g_dtype != "f32":
        raise ValueError(g_dtype)
    return g


def numpy_matrix(w: Workload, idx: int, step: int = 0) -> dict:
    """Gradient of matrix ``idx`` at ``step`` and its initial weights."""
    spec = w.matrices[idx]
    g = numpy_gradient(spec.rows, spec.cols, w.rank, w.noise, w.g_dtype, [w.wid, idx, step, 0])
    w0 = (0.02 * _rng(w.wid, idx, 0, 1).standard_normal((spec.rows, spec.cols))).astype(np.float32)
    return {"G": g, "W0": w0, "B0": np.zeros((spec.rows, spec.cols), np.float32)}


def gradient_as_f64(g: np.ndarray, g_dtype: str) -> np.ndarray:
    """Exact float64 view of a generated gradient (bf16 bits are widened exactly)."""
    if g_dtype == "bf16":
        return bf16_bits_to_f32(g).astype(np.float64)
    return np.asarray(g, dtype=np.float64)


# ---------------------------------------------------------------- torch side
def torch_matrix(w: Workload, idx: int, step: int, device, generator=None) -> dict:
    """Same recipe on a torch device (float32 draws); for full-size workloads."""
    import torch

    spec = w.matrices[idx]
    gen = generator
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(((w.wid * 1_000_003 + idx) * 1_000_033 + step) & 0x7FFFFFFFFFFF)
    p = torch.randn(spec.rows, w.rank, device=device, generator=gen)
    q = torch.randn(w.rank, spec.cols, device=device, generator=gen)
    g = torch.randn(spec.rows, spec.cols, device=device, generator=gen)
    g.mul_(w.noise).add_(p @ q, alpha=0.25)
    if w.g_dtype == "bf16":
        g = g.to(torch.bfloat16)
    w0 = torch.randn(spec.rows, spec.cols, device=device, generator=gen).mul_(0.02)
    return {"G": g, "W0": w0, "B0": torch.zeros_like(w0)}


# ---------------------------------------------------------------- special inputs
def signed_partial_permutation_entries(rows: int, cols: int, count: int, seed: Sequence[int]):
    """Row indices, column indices and signs of ``signed_partial_permutation``
    (for building the matrix where it lives, e.g. on the GPU at large sizes)."""
    if count > min(rows, cols):
        raise ValueError("count exceeds min(rows, cols)")
    rng = np.random.default_rng(list(seed))
    r = rng.permutation(rows)[:count]
    c = rng.permutation(cols)[:count]
    s = rng.choice(np.array([-1.0, 1.0]), size=count)
    return r, c, s


def signed_partial_permutation(rows: int, cols: int, count: int, seed: Sequence[int]) -> np.ndarray:
    """``count`` entries of +-1 at distinct positions, no two in one row or column."""
    r, c, s = signed_partial_permutation_entries(rows, cols, count, seed)
    m = np.zeros((rows, cols), np.float32)
    m[r, c] = s
    return m


def sparse_signs(rows: int, cols: int, count: int, seed: Sequence[int]) -> np.ndarray:
    """``count`` entries of +-1 at distinct random positions (rows/cols may repeat)."""
    if count > rows * cols:
        raise ValueError("count exceeds rows * cols")
    rng = np.random.default_rng(list(seed))
    pos = rng.choice(rows * cols, size=count, replace=False)
    s = rng.choice(np.array([-1.0, 1.0]), size=count)
    m = np.zeros(rows * cols, np.float32)
    m[pos] = s
    return m.reshape(rows, cols)
