"""Pins for the oracle's quantised-activation product (``xq`` on the q8 ops).

The decode lane of the emit.rs page quantises an activation row to Q8_0 (the
`lk_quant` launch: blocks of 32 values with one scale each) before its Q8_0
GEMV.  The pages do not print the quantiser's arithmetic; the reading pinned
here is the symmetric absmax form: per block d = amax / 127, each code the
quotient x / d rounded to the nearest integer with ties to even, and the
product sums, block by block, the exact integer dot product of the codes
weighted by d times the weight's block scale.

Expected values come from closed forms on inputs where every step is exact,
from integer arithmetic, or from the quantisation error bound -- never from
the oracle itself.
"""
import numpy as np
import pytest

from persistent_whole_step_amd.programs import Program


def _prog(m, k, n, xq=True, bias=False):
    p = Program()
    x = p.input("x", "f32", (m, k))
    q = p.input("q", "i8", (n, k))
    s = p.input("s", "f32", (n, (k + 31) // 32))
    args = [x, q, s]
    if bias:
        b = p.input("b", "f32", (n,))
        args = [b] + args
    attrs = {"xq": 1.0} if xq else {}
    p.output(p.op("addmm_q8" if bias else "mm_q8", args, "f32", (m, n), **attrs))
    return p


def _one_hot(k):
    """Weights that pick activation element c into output c (scales 1)."""
    q = np.eye(k, dtype=np.int8)
    s = np.ones((k, (k + 31) // 32), np.float32)
    return q, s


def test_unit_scale_blocks_give_the_integers_back(oracle_mod):
    # amax = 127 in every block: d = 1 exactly, codes = x for integer x
    k = 64
    rng = np.random.default_rng(0)
    x = rng.integers(-126, 127, (2, k)).astype(np.float32)
    x[:, 5] = 127.0
    x[:, 40] = -127.0
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(2, k, k).text(), [x, q, s])
    np.testing.assert_array_equal(y, x)


def test_ties_round_to_even(oracle_mod):
    k = 32
    x = np.zeros((1, k), np.float32)
    x[0, 0] = 127.0  # d = 1
    x[0, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(1, k, k).text(), [x, q, s])
    np.testing.assert_array_equal(y[0, 1:9], np.float32([2, 4, -2, -4, 0, -0.0, 2, 126]))


def test_power_of_two_scale_and_integer_dot(oracle_mod):
    # amax = 127 * 2^-3 -> d = 2^-3; x = code * 2^-3 exactly; weights random
    # integers with power-of-two block scales: the result is exact and equals
    # the integer dot product times the scales
    m, k, n = 3, 96, 7
    rng = np.random.default_rng(1)
    codes = rng.integers(-127, 128, (m, k))
    codes[:, ::32] = 127  # every block reaches the maximum code
    x = (codes * 2.0 ** -3).astype(np.float32)
    q = rng.integers(-127, 128, (n, k)).astype(np.int8)
    s = (2.0 ** rng.integers(-8, 0, (n, k // 32))).astype(np.float32)
    want = np.zeros((m, n))
    for b in range(k // 32):
        sl = slice(32 * b, 32 * b + 32)
        want += (codes[:, sl] @ q[:, sl].astype(np.int64).T) * (2.0 ** -3) * s[:, b][None, :]
    (y,) = oracle_mod.run(_prog(m, k, n).text(), [x, q, s])
    np.testing.assert_array_equal(y.astype(np.float64), want)


def test_matches_plain_product_when_codes_are_the_values(oracle_mod):
    # integer activations with amax 127 per block: quantisation is the
    # identity, so the xq product equals the unquantised one (both exact)
    m, k, n = 2, 64, 5
    rng = np.random.default_rng(2)
    x = rng.integers(-100, 101, (m, k)).astype(np.float32)
    x[:, 0] = 127.0
    x[:, 33] = -127.0
    q = rng.integers(-127, 128, (n, k)).astype(np.int8)
    s = (2.0 ** rng.integers(-6, 0, (n, 2))).astype(np.float32)
    b = rng.integers(-50, 50, n).astype(np.float32)
    (yq,) = oracle_mod.run(_prog(m, k, n, bias=True).text(), [x, q, s, b])
    (yp,) = oracle_mod.run(_prog(m, k, n, xq=False, bias=True).text(), [x, q, s, b])
    np.testing.assert_array_equal(yq, yp)


def test_zero_block_and_block_independence(oracle_mod):
    # block 0 all zero (d = 0, codes 0); a huge value in block 1 does not
    # change block 2's scale
    k = 96
    x = np.zeros((1, k), np.float32)
    x[0, 32] = 1.0e6
    x[0, 33] = 1.0
    x[0, 64] = 127.0
    x[0, 65] = 3.0
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(1, k, k).text(), [x, q, s])
    assert np.all(y[0, :32] == 0)
    assert y[0, 64] == 127.0 and y[0, 65] == 3.0
    assert y[0, 33] == 0.0  # 1 is far below half a step of 1e6 / 127
    # the block's largest element is represented by code 127 exactly
    d = np.float32(1.0e6) / np.float32(127)
    assert y[0, 32] == np.float32(d * np.float32(127))


@pytest.mark.parametrize("k", [40, 100, 4096])
def test_quantisation_error_at_most_half_a_step(oracle_mod, k):
    # one-hot weights return d * code for each element: within half a
    # quantisation step of x (plus the rounding of the product), the largest
    # element of each block reproduced to within one rounding
    rng = np.random.default_rng(k)
    x = (rng.standard_normal((2, k)) * 10.0 ** rng.uniform(-3, 3, (2, 1))).astype(np.float32)
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(2, k, k).text(), [x, q, s])
    for r in range(2):
        for b in range((k + 31) // 32):
            sl = slice(32 * b, min(k, 32 * b + 32))
            xb = x[r, sl].astype(np.float64)
            amax = np.abs(xb).max()
            d = amax / 127.0
            err = np.abs(y[r, sl].astype(np.float64) - xb)
            assert np.all(err <= d / 2 * (1 + 1e-5) + np.abs(xb) * 2.0 ** -23)
            j = np.argmax(np.abs(xb))
            assert abs(y[r, sl][j] - xb[j]) <= abs(xb[j]) * 2.0 ** -22


def test_ragged_last_block(oracle_mod):
    # k = 40: a full block and one of 8; the short block's scale is its own
    k = 40
    x = np.zeros((1, k), np.float32)
    x[0, 0] = 127.0
    x[0, 32] = 254.0  # d = 2 for the short block
    x[0, 33] = 5.0    # 5 / 2 = 2.5 -> 2 (ties to even) -> 4
    x[0, 34] = -7.0   # -3.5 -> -4 -> -8
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(1, k, k).text(), [x, q, s])
    np.testing.assert_array_equal(y[0, 32:35], np.float32([254, 4, -8]))


def test_xq_rejected_outside_q8(oracle_mod):
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (3, 4))
    p.output(p.op("mm", [a, b], "f32", (2, 4), xq=1.0))
    with pytest.raises(Exception):
        oracle_mod.run(p.text(), [np.ones((2, 3), np.float32), np.ones((3, 4), np.float32)])


def test_parity_harness_codes_match_oracle(oracle_mod):
    """The parity harness's own float32 quantiser (used for the tolerance
    reference of GPU results) gives the oracle's codes and scales."""
    from tests import parity
    k = 1000
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, k)) * 3).astype(np.float32)
    x[1, :32] = 0
    q, s = _one_hot(k)
    (y,) = oracle_mod.run(_prog(3, k, k).text(), [x, q, s])
    codes, d = parity.xq_codes(x)
    want = (np.repeat(d, 32, axis=1)[:, :k] * codes.astype(np.float32)).astype(np.float32)
    np.testing.assert_array_equal(y, want)
