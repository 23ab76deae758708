"""ctypes wrapper of the CPU oracle (test infrastructure only).

``run(text, inputs)`` evaluates a ``tkir 1`` program on host numpy arrays in
storage form (float32, float16, uint16 bf16 bits, int8) and returns the
outputs in storage form.  ``run64`` evaluates the same program in binary64
with every buffer a float64 array (finite-difference checks).
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

from .build import LIB, build

_lib = None
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i8": np.int8}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        l = ctypes.CDLL(LIB)
        l.oracle_run.restype = ctypes.c_int
        l.oracle_run.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int]
        l.oracle_error.restype = ctypes.c_char_p
        l.oracle_threads.restype = ctypes.c_int
        l.oracle_set_threads.restype = None
        l.oracle_set_threads.argtypes = [ctypes.c_int]
        for name in ("oracle_round_bf16", "oracle_round_f16"):
            f = getattr(l, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        _lib = l
    return _lib


class OracleError(RuntimeError):
    pass


def _dims(s: str):
    return () if s == "-" else tuple(int(v) for v in s.split("x"))


def output_specs(text: str):
    """(shape, dtype) of each ``out`` statement, read from the program text."""
    outs = []
    for line in text.splitlines():
        tok = line.split(";")[0].split()
        if tok and tok[0] == "out":
            _, dtype, shape, _, _ = tok[1].split(":")
            outs.append((_dims(shape), dtype))
    return outs


def input_count(text: str) -> int:
    return sum(1 for line in text.splitlines() if line.split(";")[0].split()[:1] == ["in"])


def _call(text: str, ins, outs, mode: int):
    l = lib()
    in_ptrs = (ctypes.c_void_p * max(1, len(ins)))(*[a.ctypes.data for a in ins])
    out_ptrs = (ctypes.c_void_p * max(1, len(outs)))(*[a.ctypes.data for a in outs])
    rc = l.oracle_run(text.encode(), in_ptrs, len(ins), out_ptrs, len(outs), mode)
    if rc != 0:
        raise OracleError(l.oracle_error().decode())


def run(text: str, inputs, outputs=None):
    """Evaluate in float32 with per-op rounding.  ``outputs`` (optional) are
    preallocated arrays; an in-place slot may be the very input array."""
    ins = [np.ascontiguousarray(a) if not a.flags["C_CONTIGUOUS"] else a for a in inputs]
    if outputs is None:
        outputs = [np.empty(shape, dtype=_NP[dt]) for shape, dt in output_specs(text)]
    _call(text, ins, outputs, 0)
    return outputs


def run64(text: str, inputs):
    ins = [np.ascontiguousarray(a, dtype=np.float64) for a in inputs]
    outs = [np.empty(shape, dtype=np.float64) for shape, _ in output_specs(text)]
    _call(text, ins, outs, 1)
    return outs


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops (results do not depend on it)."""
    lib().oracle_set_threads(int(n))


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_round_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def round_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_round_f16(x.ctypes.data, out.ctypes.data, x.size)
    return out
