"""Pins for the oracle's per-op semantics (trainkernel pages, codegen.py:
`point_expr`, `emit_mm`, `emit_reduction`, `read`/`operand` for views and
broadcasting, and the device helpers `mk_relu` / `mk_square`).

Every expected value here comes from IEEE-754 arithmetic on values where the
result is exact, from integer arithmetic, from a closed form, or from an
independent library computation -- never from the oracle itself.
"""
import math

import numpy as np
import pytest

from persistent_whole_step_amd.programs import Program, Spec, f32
from persistent_whole_step_amd import synth


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def run1(oracle_mod, prog, inputs):
    return oracle_mod.run(prog.text(), inputs)


def unary_prog(opcode, dtype="f32", n=8, **attrs):
    p = Program()
    x = p.input("x", dtype, (n,))
    y = p.op(opcode, [x], dtype, **attrs)
    p.output(y)
    return p


def binary_prog(opcode, n=8, dtype="f32", **attrs):
    p = Program()
    a = p.input("a", dtype, (n,))
    b = p.input("b", dtype, (n,))
    y = p.op(opcode, [a, b], dtype, **attrs)
    p.output(y)
    return p


# ----------------------------------------------------------------- pointwise

def test_relu_special_values(oracle_mod):
    x = np.array([-0.0, 0.0, -1.5, 2.5, np.inf, -np.inf, np.nan, -1e-45], dtype=np.float32)
    (y,) = run1(oracle_mod, unary_prog("relu"), [x])
    # relu is `x < 0 ? 0 : x`: -0 is not < 0 so it passes through with its sign.
    assert bits(y[0]) == 0x80000000
    assert bits(y[1]) == 0
    assert y[2] == 0 and bits(y[2]) == 0
    assert y[3] == 2.5 and y[4] == np.inf and y[5] == 0
    assert np.isnan(y[6])
    assert bits(y[7]) == 0  # negative subnormal is < 0


def test_threshold_backward_masks_on_input(oracle_mod):
    p = Program()
    g = p.input("g", "f32", (8,))
    x = p.input("x", "f32", (8,))
    y = p.op("threshold_backward", [g, x], "f32", threshold=0.0)
    p.output(y)
    gv = np.arange(1, 9, dtype=np.float32)
    xv = np.array([-0.0, 0.0, -3.0, 1e-45, np.nan, 5.0, -np.inf, np.inf], dtype=np.float32)
    (out,) = run1(oracle_mod, p, [gv, xv])
    # x <= 0 (including -0) -> 0; NaN compares false -> g passes.
    np.testing.assert_array_equal(out, np.array([0, 0, 0, 4, 5, 6, 0, 8], dtype=np.float32))


def test_threshold_nonzero(oracle_mod):
    p = Program()
    g = p.input("g", "f32", (4,))
    x = p.input("x", "f32", (4,))
    p.output(p.op("threshold_backward", [g, x], "f32", threshold=1.5))
    (out,) = run1(oracle_mod, p, [np.full(4, 7, np.float32), np.array([1.0, 1.5, 1.75, 3.0], np.float32)])
    np.testing.assert_array_equal(out, [0, 0, 7, 7])


def test_pow_two_is_square_bitexact(oracle_mod):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(4096) * 1e3).astype(np.float32)
    p = Program()
    a = p.input("a", "f32", (4096,))
    p.output(p.op("pow", [a, 2.0], "f32"))
    (y,) = run1(oracle_mod, p, [x])
    np.testing.assert_array_equal(bits(y), bits(x * x))


def test_pow_other_exponent_close_to_libm(oracle_mod):
    x = np.array([0.5, 2.0, 3.0, 10.0], dtype=np.float32)
    p = Program()
    a = p.input("a", "f32", (4,))
    p.output(p.op("pow", [a, 3.0], "f32"))
    (y,) = run1(oracle_mod, p, [x])
    np.testing.assert_array_equal(y, [0.125, 8.0, 27.0, 1000.0])  # exact cubes


def test_add_sub_alpha_and_operand_order(oracle_mod):
    a = np.array([5.0, 1.0, -2.0, 0.5], np.float32)
    b = np.array([3.0, 4.0, 0.25, -8.0], np.float32)
    (s,) = run1(oracle_mod, binary_prog("sub", n=4, alpha=2.0), [a, b])
    np.testing.assert_array_equal(s, a - 2 * b)  # exact on these dyadics: 5-6, 1-8, ...
    (ad,) = run1(oracle_mod, binary_prog("add", n=4, alpha=0.5), [a, b])
    np.testing.assert_array_equal(ad, [6.5, 3.0, -1.875, -3.5])
    (d,) = run1(oracle_mod, binary_prog("div", n=4), [a, b])
    assert bits(d[0]) == 0x3FD55555  # 5/3 to nearest float32
    np.testing.assert_array_equal(d[1:], [0.25, -8.0, -0.0625])


def test_add_alpha_rounds_product_then_sum(oracle_mod):
    # a + fl(alpha*b), two roundings, no fused multiply-add.  With
    # alpha = b = 1 + 2^-12 the product 1 + 2^-11 + 2^-24 rounds (tie, even)
    # to 1 + 2^-11, so -1 + it is exactly 2^-11; a fused form would give
    # 2^-11 + 2^-24.
    (y,) = run1(oracle_mod, binary_prog("add", n=1, alpha=1.0 + 2 ** -12),
                [np.array([-1.0], np.float32), np.array([1.0 + 2 ** -12], np.float32)])
    assert y[0] == np.float32(2 ** -11)


def test_division_correctly_rounded_known_value(oracle_mod):
    (y,) = run1(oracle_mod, binary_prog("div", n=2), [np.array([1.0, 2.0], np.float32), np.array([3.0, 3.0], np.float32)])
    assert bits(y[0]) == 0x3EAAAAAB  # 1/3 to nearest float32
    assert bits(y[1]) == 0x3F2AAAAB  # 2/3 to nearest float32


def test_neg_full_cast(oracle_mod):
    x = np.array([0.0, -0.0, 1.5, np.inf], np.float32)
    (y,) = run1(oracle_mod, unary_prog("neg", n=4), [x])
    np.testing.assert_array_equal(bits(y), [0x80000000, 0, bits(-1.5), bits(-np.inf)])
    p = Program()
    a = p.input("a", "f32", (3,))
    p.output(p.op("full", [], "f32", shape=(2, 3), value=2.75))
    p.output(p.op("cast", [a], "bf16"))
    p.output(p.op("cast", [a], "f16"))
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65520.0], np.float32)
    full, cb, ch = run1(oracle_mod, p, [v])
    np.testing.assert_array_equal(full, np.full((2, 3), 2.75, np.float32))
    np.testing.assert_array_equal(cb, [0x3F80, 0x3F82, 0x4780])  # ties to even; 65520 -> 65536 in bf16
    assert ch[2] == np.inf and ch[0] == np.float16(1.0 + 2 ** -8)  # exact in f16


def test_per_op_rounding_in_chain(oracle_mod):
    # bf16 chain: each op rounds.  1 + 2^-8 is not a bf16 value: mul by 1 rounds
    # it to 1.0, so the following sub by 1 gives exactly 0 (not 2^-8).
    p = Program()
    a = p.input("a", "f32", (1,))
    one = p.input("one", "f32", (1,))
    m = p.op("mul", [a, one], "bf16")
    s = p.op("sub", [m, one], "f32")
    p.output(s)
    (y,) = run1(oracle_mod, p, [np.array([1.0 + 2 ** -8], np.float32), np.array([1.0], np.float32)])
    assert y[0] == 0.0


def test_broadcast_rows_cols_scalar_and_views(oracle_mod):
    p = Program()
    m = p.input("m", "f32", (2, 3))
    r = p.input("r", "f32", (3,))
    c = p.input("c", "f32", (2, 1))
    p.output(p.op("add", [m, r], "f32"))
    p.output(p.op("mul", [m, c], "f32"))
    p.output(p.op("sub", [m, 1.5], "f32"))
    # transposed view of m read as [3,2], and an offset view of its 2nd row
    p.output(p.op("cast", [m.T], "f32", shape=(3, 2)))
    p.output(p.op("cast", [m.view((3,), (1,), 3)], "f32", shape=(3,)))
    mv = np.arange(6, dtype=np.float32).reshape(2, 3)
    rv = np.array([10, 20, 30], np.float32)
    cv = np.array([[2], [-1]], np.float32)
    o1, o2, o3, o4, o5 = run1(oracle_mod, p, [mv, rv, cv])
    np.testing.assert_array_equal(o1, mv + rv)
    np.testing.assert_array_equal(o2, mv * cv)
    np.testing.assert_array_equal(o3, mv - 1.5)
    np.testing.assert_array_equal(o4, mv.T)
    np.testing.assert_array_equal(o5, mv[1])


def test_output_view_and_dtype_conversion(oracle_mod):
    p = Program()
    a = p.input("a", "f32", (2, 2))
    y = p.op("mul", [a, 1.0], "f32")
    p.outputs.append(Spec(y.buf, "bf16", (2, 2), (1, 2), 0))  # transposed, converted
    (o,) = run1(oracle_mod, p, [np.array([[1.0, 1.0 + 2 ** -8], [3.0, 4.0]], np.float32)])
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(o), [[1.0, 3.0], [1.0, 4.0]])


# --------------------------------------------------------------- contractions

def mm_prog(m, k, n, dtype="f32", ta=False, tb=False, bias=None, **attrs):
    p = Program()
    A = p.input("A", dtype, (k, m) if ta else (m, k))
    B = p.input("B", dtype, (n, k) if tb else (k, n))
    av = A.T if ta else A
    bv = B.T if tb else B
    if bias is None:
        y = p.op("mm", [av, bv], dtype, (m, n), **attrs)
    else:
        bi = p.input("bias", dtype, bias)
        y = p.op("addmm", [bi, av, bv], dtype, (m, n), **attrs)
    p.output(y)
    return p


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_integer_matmul_exact(oracle_mod, ta, tb):
    rng = np.random.default_rng(2)
    m, k, n = 7, 33, 5
    A = rng.integers(-8, 9, size=(m, k))
    B = rng.integers(-8, 9, size=(k, n))
    Ai = (A.T if ta else A).astype(np.float32).copy()
    Bi = (B.T if tb else B).astype(np.float32).copy()
    (y,) = run1(oracle_mod, mm_prog(m, k, n, ta=ta, tb=tb), [Ai, Bi])
    np.testing.assert_array_equal(y, (A @ B).astype(np.float32))


def test_addmm_alpha_beta_cases(oracle_mod):
    rng = np.random.default_rng(3)
    m, k, n = 4, 6, 3
    A = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
    B = rng.integers(-4, 5, size=(k, n)).astype(np.float32)
    bias = np.array([1.0, -2.0, 0.5], np.float32)
    ref = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    for alpha, beta, want in [
        (1.0, 1.0, ref + bias),
        (2.0, 0.5, 2 * ref + 0.5 * bias),
        (0.0, 0.0, np.zeros_like(ref)),
        (0.25, 0.0, 0.25 * ref),
        (0.0, -1.0, np.broadcast_to(-bias, ref.shape)),
    ]:
        (y,) = run1(oracle_mod, mm_prog(m, k, n, bias=(n,), alpha=alpha, beta=beta), [A, B, bias])
        np.testing.assert_array_equal(y, want.astype(np.float32))
    # beta == 0 never reads the bias: a NaN bias does not leak
    (y,) = run1(oracle_mod, mm_prog(m, k, n, bias=(n,), alpha=1.0, beta=0.0), [A, B, np.full(3, np.nan, np.float32)])
    np.testing.assert_array_equal(y, ref.astype(np.float32))
    # alpha == 0 never uses the product: an Inf operand does not leak
    Ainf = A.copy()
    Ainf[0, 0] = np.inf
    (y,) = run1(oracle_mod, mm_prog(m, k, n, bias=(n,), alpha=0.0, beta=1.0), [Ainf, B, bias])
    np.testing.assert_array_equal(y, np.broadcast_to(bias, ref.shape))


def test_matmul_higham_bound(oracle_mod):
    rng = np.random.default_rng(4)
    m, k, n = 9, 777, 11
    A = rng.standard_normal((m, k)).astype(np.float32)
    B = rng.standard_normal((k, n)).astype(np.float32)
    (y,) = run1(oracle_mod, mm_prog(m, k, n), [A, B])
    exact = A.astype(np.float64) @ B.astype(np.float64)
    mag = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    assert np.all(np.abs(y - exact) <= gamma * mag)


def test_matmul_sequential_fma_order(oracle_mod):
    # acc = fma(a, b, acc) from +0 in k order: with a = [2^24, 1, -2^24] and
    # b = 1, the sequential sum is (2^24 + 1) -> 2^24 (tie to even), then 0.
    A = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]], np.float32)
    B = np.ones((3, 1), np.float32)
    (y,) = run1(oracle_mod, mm_prog(1, 3, 1), [A, B])
    assert y[0, 0] == 0.0
    # fma keeps the exact product: acc = -1, then fma((1+2^-12)^2, -1) is
    # exactly 2^-11 + 2^-24 (a rounded product would give 2^-11)
    A = np.array([[1.0, 1.0 + 2 ** -12]], np.float32)
    B = np.array([[-1.0], [1.0 + 2 ** -12]], np.float32)
    (y,) = run1(oracle_mod, mm_prog(1, 2, 1), [A, B])
    assert y[0, 0] == np.float32(2 ** -11 + 2 ** -24)


def test_bf16_matmul_output_rounded(oracle_mod):
    A = synth._to_storage(np.array([[1.0, 2.0 ** -8]]), "bf16")
    B = synth._to_storage(np.array([[1.0], [1.0]]), "bf16")
    (y,) = run1(oracle_mod, mm_prog(1, 2, 1, dtype="bf16"), [A, B])
    assert int(y[0, 0]) == 0x3F80  # 1 + 2^-8 -> ties to even -> 1.0


@pytest.mark.parametrize("m", [1, 3])
def test_q8_contraction_exact_with_power_of_two_scales(oracle_mod, m):
    rng = np.random.default_rng(5)
    k, n = 96, 7
    nb = (k + 31) // 32
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = (2.0 ** rng.integers(-6, 1, size=(n, nb))).astype(np.float32)
    x = rng.integers(-3, 4, size=(m, k)).astype(np.float32)
    b = np.array(rng.integers(-5, 6, size=n), np.float32)
    p = Program()
    xi = p.input("x", "f32", (m, k))
    qi = p.input("q", "i8", (n, k))
    si = p.input("s", "f32", (n, nb))
    bi = p.input("b", "f32", (n,))
    p.output(p.op("addmm_q8", [bi, xi, qi, si], "f32", (m, n)))
    (y,) = run1(oracle_mod, p, [x, q, s, b])
    W = q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)[:, :k]
    np.testing.assert_array_equal(y, (x.astype(np.float64) @ W.T + b).astype(np.float32))


# ----------------------------------------------------------------- reductions

def red_prog(shape, dims, opcode="sum", out_shape=None, dtype="f32"):
    p = Program()
    x = p.input("x", dtype, shape)
    if out_shape is None:
        if dims is None:
            out_shape = ()
        else:
            nd = len(shape)
            red = {d % nd for d in dims}
            out_shape = tuple(s for i, s in enumerate(shape) if i not in red)
    p.output(p.op(opcode, [x], dtype, out_shape, dims=dims))
    return p


@pytest.mark.parametrize("dims", [None, [0], [1], [-1], [0, 2], [2, 0, -3]])
def test_integer_sums_exact(oracle_mod, dims):
    rng = np.random.default_rng(6)
    x = rng.integers(-50, 51, size=(3, 4, 5)).astype(np.float32)
    (y,) = run1(oracle_mod, red_prog((3, 4, 5), dims), [x])
    axes = None if dims is None else tuple(sorted({d % 3 for d in dims}))
    np.testing.assert_array_equal(y, x.astype(np.int64).sum(axis=axes).astype(np.float32))


def test_large_sum_covers_every_element(oracle_mod):
    n = 300_000  # far above 131072, the most a 256 x 512 partial split could cover
    x = np.ones(n, np.float32)
    (y,) = run1(oracle_mod, red_prog((n,), None), [x])
    assert y == n
    (m,) = run1(oracle_mod, red_prog((n,), None, "mean"), [np.full(n, 0.375, np.float32)])
    assert m == 0.375


def test_mean_of_constant_and_empty(oracle_mod):
    (m,) = run1(oracle_mod, red_prog((6, 7), None, "mean"), [np.full((6, 7), -2.5, np.float32)])
    assert m == -2.5
    (s,) = run1(oracle_mod, red_prog((0, 3), [0]), [np.zeros((0, 3), np.float32)])
    np.testing.assert_array_equal(s, [0, 0, 0])
    (e,) = run1(oracle_mod, red_prog((0,), None, "mean"), [np.zeros((0,), np.float32)])
    assert np.isnan(e)


def test_column_sum_keepdim_shape(oracle_mod):
    x = np.arange(12, dtype=np.float32).reshape(3, 4)
    (y,) = run1(oracle_mod, red_prog((3, 4), [0], out_shape=(1, 4)), [x])
    np.testing.assert_array_equal(y, x.sum(0, keepdims=True))


# ---------------------------------------------------------------- diagnostics

@pytest.mark.parametrize("mutate,needle", [
    (lambda t: t.replace("#0x1.0000000000000p+1", "#inf"), "non-finite"),
    (lambda t: t.replace(" mul ", " tanh "), "unsupported pointwise"),
    (lambda t: t.replace("tkir 1", "tkir 2"), "header"),
])
def test_oracle_rejects(oracle_mod, mutate, needle):
    p = Program()
    a = p.input("a", "f32", (4,))
    p.output(p.op("mul", [a, 2.0], "f32", name="y"))
    with pytest.raises(oracle_mod.OracleError, match=needle):
        oracle_mod.run(mutate(p.text()), [np.zeros(4, np.float32)])


def test_oracle_rejects_bad_shapes(oracle_mod):
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (4,))
    p.output(p.op("add", [a, b], "f32"))
    with pytest.raises(oracle_mod.OracleError, match="broadcast"):
        oracle_mod.run(p.text(), [np.zeros((2, 3), np.float32), np.zeros(4, np.float32)])
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (4, 2))
    p.output(p.op("mm", [a, b], "f32", (2, 2)))
    with pytest.raises(oracle_mod.OracleError, match="compatible"):
        oracle_mod.run(p.text(), [np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32)])
