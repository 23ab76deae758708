"""Pins for the oracle's float32 -> bf16 / f16 round-to-nearest-even.

The trainkernel pages round every low-precision value with the `_rn`
conversions (codegen.py, `_round` and `store`).  The oracle writes that
rounding out from the IEEE-754 roundTiesToEven definition; here it is checked
over all 2^32 float32 bit patterns against library conversions (numpy's
float32->float16 cast and torch's CPU float32->bfloat16 cast, both RNE), and
on hand-picked cases whose results follow from the definition alone.
"""
import os

import numpy as np
import pytest
import torch

EXHAUSTIVE = os.environ.get("TK_EXHAUSTIVE") == "1"


def _is_nan16(h, exp_mask, man_mask):
    return ((h & exp_mask) == exp_mask) & ((h & man_mask) != 0)


def _library_round(x, fmt):
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_structured_sweep(oracle_mod, fmt):
    """Every value of the top 19 bits (sign, exponent, leading mantissa) with
    the low 13 bits set to each pattern that decides a rounding (0, 1, just
    below/at/above the half-way point for both formats, all ones) plus random
    fills: the part of the full sweep that runs in seconds."""
    rng = np.random.default_rng(7)
    low = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF, 0x7FFF & 0x1FFF] +
                   list(rng.integers(0, 1 << 13, 9)), dtype=np.uint32)
    high = np.arange(1 << 19, dtype=np.uint32) << 13
    bits = (high[:, None] | low[None, :]).ravel()
    # bf16's decision bits are the low 16: add patterns around 0x8000 there
    low16 = np.array([0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = np.concatenate([bits, ((np.arange(1 << 16, dtype=np.uint32) << 16)[:, None] | low16[None, :]).ravel()])
    x = bits.view(np.float32)
    got = oracle_mod.round_f16(x) if fmt == "f16" else oracle_mod.round_bf16(x)
    ref = _library_round(x, fmt)
    masks = (0x7C00, 0x03FF) if fmt == "f16" else (0x7F80, 0x007F)
    idx = np.flatnonzero(got != ref)
    idx = idx[~(_is_nan16(got[idx], *masks) & _is_nan16(ref[idx], *masks))]
    assert idx.size == 0, [(hex(int(bits[i])), hex(int(got[i])), hex(int(ref[i]))) for i in idx[:5]]


@pytest.mark.slow
@pytest.mark.skipif(not EXHAUSTIVE, reason="full 2^32 sweep takes minutes; set TK_EXHAUSTIVE=1")
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_exhaustive_all_float32_patterns(oracle_mod, fmt):
    import ctypes
    lib = oracle_mod.lib()
    lib.oracle_iota_bits.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int64]
    chunk = 1 << 26
    buf = np.empty(chunk, np.uint32)
    bad, first = 0, None
    masks = (0x7C00, 0x03FF) if fmt == "f16" else (0x7F80, 0x007F)
    for lo in range(0, 1 << 32, chunk):
        lib.oracle_iota_bits(lo, buf.ctypes.data, chunk)
        x = buf.view(np.float32)
        if fmt == "f16":
            got = oracle_mod.round_f16(x)
            ref = x.astype(np.float16).view(np.uint16)
        else:
            got = oracle_mod.round_bf16(x)
            ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        idx = np.flatnonzero(got != ref)
        if idx.size:
            # NaN results compare equal whatever their payload
            both_nan = _is_nan16(got[idx], *masks) & _is_nan16(ref[idx], *masks)
            idx = idx[~both_nan]
        if idx.size and first is None:
            i = int(idx[0])
            first = (hex(int(buf[i])), hex(int(got[i])), hex(int(ref[i])))
        bad += int(idx.size)
    assert bad == 0, f"{bad} mismatches, first {first}"


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


# (float32 bits, expected bf16 bits): each row follows from the definition.
BF16_CASES = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway between 1 and 1+2^-7, ties to even (1.0)
    (0x3F818000, 0x3F82),  # 1 + 3*2^-8: halfway, ties to even (1 + 2^-6)
    (0x3F808001, 0x3F81),  # just above halfway rounds up
    (0x7F7FFFFF, 0x7F80),  # FLT_MAX rounds past the largest bf16 -> +Inf
    (0x7F7F7FFF, 0x7F7F),  # just below the overflow midpoint stays finite
    (0x80000000, 0x8000),  # -0 keeps its sign
    (0x00000001, 0x0000),  # smallest float32 subnormal underflows to +0
    (0x00010000, 0x0001),  # a bf16 subnormal is exact
    (0x00018000, 0x0002),  # halfway between bf16 subnormals 1 and 2 -> even (2)
    (0xFF800000, 0xFF80),  # -Inf
]

# (float32 value, expected f16 bits)
F16_CASES = [
    (1.0, 0x3C00),
    (65504.0, 0x7BFF),                # largest half
    (65519.99609375, 0x7BFF),         # below the overflow midpoint 65520
    (65520.0, 0x7C00),                # midpoint ties to even -> Inf
    (2.0 ** -24, 0x0001),             # smallest half subnormal
    (2.0 ** -25, 0x0000),             # halfway between 0 and 2^-24 -> even (0)
    (3 * 2.0 ** -26, 0x0001),         # 0.75 * 2^-24 rounds up to 2^-24
    (3 * 2.0 ** -25, 0x0002),         # 1.5 * 2^-24 ties to even -> 2 * 2^-24
    (2.0 ** -14, 0x0400),             # smallest normal
    (2.0 ** -14 - 2.0 ** -25, 0x0400),  # 1023.5 subnormal units ties to even -> 1024 (normal)
    (-0.0, 0x8000),
    (1.0 + 2.0 ** -11, 0x3C00),       # halfway above 1, ties to even
    (1.0 + 3 * 2.0 ** -11, 0x3C02),   # halfway, ties to even (up)
]


def test_bf16_definition_cases(oracle_mod):
    for bits, want in BF16_CASES:
        got = int(oracle_mod.round_bf16(_f32(bits))[0])
        assert got == want, (hex(bits), hex(got), hex(want))


def test_f16_definition_cases(oracle_mod):
    for value, want in F16_CASES:
        got = int(oracle_mod.round_f16(np.array([value], dtype=np.float32))[0])
        assert got == want, (value, hex(got), hex(want))


def test_nan_stays_nan(oracle_mod):
    for bits in (0x7FC00000, 0x7F800001, 0xFFC12345, 0x7FBFFFFF):
        b = int(oracle_mod.round_bf16(_f32(bits))[0])
        h = int(oracle_mod.round_f16(_f32(bits))[0])
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F)
        assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF)


# ------------------------------------------------------------ widening --
# Every bf16 / f16 value the oracle reads (a program input, or an op's result
# held at its dtype's precision) is widened to float32.  These pins compare the
# oracle's widening of all 65,536 bit patterns of each format with conversions
# that do not share its code: numpy's float16 -> float32 cast, and for bf16 the
# format's definition (its bits are the top half of a float32).

def _same_bits_or_both_nan(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    g, w = got.view(np.uint32), want.view(np.uint32)
    return (g == w) | (np.isnan(got) & np.isnan(want))


def _widen_program(dt):
    from persistent_whole_step_amd.programs import Program
    p = Program()
    x = p.input("x", dt, (1 << 16,))
    p.output(p.op("cast", [x], "f32"))
    return p


def test_widen_f16_all_patterns(oracle_mod):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    (got,) = oracle_mod.run(_widen_program("f16").text(), [h])
    want = h.astype(np.float32)
    ok = _same_bits_or_both_nan(got, want)
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, [(hex(int(h.view(np.uint16)[i])), got[i], want[i]) for i in bad[:5]]
    # the subnormal range is covered: 1023 positive and 1023 negative patterns
    sub = (h.view(np.uint16) & 0x7C00) == 0
    assert int((sub & (h.view(np.uint16) & 0x3FF != 0)).sum()) == 2046


def test_widen_bf16_all_patterns(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    (got,) = oracle_mod.run(_widen_program("bf16").text(), [bits])
    want = (bits.astype(np.uint32) << 16).view(np.float32)
    bad = np.flatnonzero(~_same_bits_or_both_nan(got, want))
    assert bad.size == 0, [(hex(int(bits[i])), got[i], want[i]) for i in bad[:5]]
    # torch's bfloat16 -> float32 conversion agrees on every non-NaN pattern
    tw = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert _same_bits_or_both_nan(got, tw).all()


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_op_results_held_at_dtype_precision(oracle_mod, dt):
    """An op whose result dtype is f16/bf16 holds the rounded value widened
    back to float32 (the value model): multiplying every finite value of the
    format by 1 and reading the result as float32 gives the value itself,
    subnormals included, and the stored result has the input's bits."""
    from persistent_whole_step_amd.programs import Program
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dt == "f16":
        x32 = bits.view(np.float16).astype(np.float32)
    else:
        x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(x32)
    x32, bits = x32[keep], bits[keep]
    p = Program()
    x = p.input("x", "f32", x32.shape)
    y = p.op("mul", [x, 1.0], dt)
    p.output(y)
    p.output(p.op("cast", [y], "f32"))
    stored, wide = oracle_mod.run(p.text(), [x32])
    assert (stored.view(np.uint16) == bits).all()
    assert (wide.view(np.uint32) == x32.view(np.uint32)).all()
