"""Seeded synthetic inputs for the whole-step programs.

This module only draws random numbers and stores them in a tensor's storage
dtype.  It holds none of the step's arithmetic, so both the CPU oracle (in the
tests) and the HIP path are fed from here without sharing any computation.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per program instance):
draws are float64, taken in program-input order, then rounded once to float32
(``ndarray.astype``) and, for 16-bit storage, once more from float32 to the
storage dtype with round-to-nearest-even (numpy for float16, torch CPU for
bfloat16).  ``N(0, v)`` names a normal with *variance* v.  Integer weights
``U{-127..127}`` are uniform integers; block scales ``U(0, 0.01]`` are drawn
as ``0.01 * (1 - u)`` with ``u`` uniform in [0, 1).

Tensors are numpy arrays in their storage form: float32 -> float32,
float16 -> float16, bfloat16 -> uint16 holding the bf16 bit pattern,
int8 -> int8.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16", "i8")


def _to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.ascontiguousarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"no float storage for dtype {dtype}")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: the 16 bits become the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of a stored tensor (all storage dtypes widen exactly)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a).astype(np.float32)


def normal(rng: np.random.Generator, shape, var: float, dtype: str) -> np.ndarray:
    return _to_storage(rng.normal(0.0, np.sqrt(var), size=shape), dtype)


def mlp_inputs(seed: int, dims, batch: int, dtype: str):
    """x, t ~ N(0,1); W_i, b_i ~ N(0, 1/fan_in).  Order: x, t, W1, b1, W2, b2, ..."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [normal(rng, (batch, dims[0]), 1.0, dtype), normal(rng, (batch, dims[-1]), 1.0, dtype)]
    for i in range(1, len(dims)):
        fan_in = dims[i - 1]
        out.append(normal(rng, (dims[i - 1], dims[i]), 1.0 / fan_in, dtype))
        out.append(normal(rng, (dims[i],), 1.0 / fan_in, dtype))
    return out


def residual_inputs(seed: int, width: int, layers: int, batch: int, dtype: str):
    """x, t ~ N(0,1); W_i, b_i ~ N(0, 0.5/width).  Order: x, t, W1, b1, ..."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [normal(rng, (batch, width), 1.0, dtype), normal(rng, (batch, width), 1.0, dtype)]
    for _ in range(layers):
        out.append(normal(rng, (width, width), 0.5 / width, dtype))
        out.append(normal(rng, (width,), 0.5 / width, dtype))
    return out


def gemv_q8_inputs(seed: int, k: int, n: int, layers: int, block: int = 32, rows: int = 1):
    """x ~ N(0,1) bf16 [rows,k]; per layer q ~ U{-127..127} int8 [n,k],
    s ~ U(0, 0.01] float32 [n, ceil(k/block)], b ~ N(0, 0.1) float32 [n].
    Layers chain, so n == k is required for more than one layer."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [normal(rng, (rows, k), 1.0, "bf16")]
    nb = (k + block - 1) // block
    for _ in range(layers):
        q = rng.integers(-127, 128, size=(n, k), dtype=np.int64).astype(np.int8)
        s = (0.01 * (1.0 - rng.random(size=(n, nb)))).astype(np.float32)
        b = normal(rng, (n,), 0.1, "f32")
        out += [q, s, b]
    return out


def adamw_state(seed: int, shapes):
    """Optimizer state part-way through training, float32: per shape, in
    order, m ~ N(0, 1e-6) then v = u^2 with u ~ N(0, 1e-6) (non-negative, as
    a running mean of squares is)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for sh in shapes:
        out.append(normal(rng, sh, 1e-6, "f32"))
        u = rng.normal(0.0, 1e-3, size=sh)
        out.append(np.ascontiguousarray(u * u).astype(np.float32))
    return out


def random_tensor(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Generic N(0, scale^2) tensor (int8: uniform integers) for small test programs."""
    if dtype == "i8":
        return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
    return _to_storage(rng.normal(0.0, scale, size=shape), dtype)
