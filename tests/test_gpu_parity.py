"""GPU parity of the persistent kernel against the CPU oracle (needs gfx950).

Each test prints its case before touching the GPU.  Sizes span several tiles
and ragged tails; pointwise-only work is compared bit for bit, contractions
and reductions under the tolerance classes of tests/parity.py, whole steps
per node with teacher forcing, and fused vs unfused schedules bitwise.
"""
import re
import sys

import numpy as np
import pytest

from persistent_whole_step_amd import programs, synth
from persistent_whole_step_amd.programs import Program

from . import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from persistent_whole_step_amd import tk
    tk.lib()


# ------------------------------------------------------------ pointwise --

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(3, 5), (64, 96), (257, 1000), (7,)])
def test_pointwise_chain_bitexact(oracle_mod, dtype, shape):
    say("pointwise", dtype, shape)
    rng = np.random.default_rng(hash((dtype, shape)) % 2 ** 32)
    p = Program()
    a = p.input("a", dtype, shape)
    b = p.input("b", dtype, shape)
    r = p.input("r", dtype, shape[-1:])
    t1 = p.op("add", [a, b], dtype, alpha=0.375)
    t2 = p.op("mul", [t1, r], dtype)
    t3 = p.op("sub", [t2, a], "f32", alpha=1.5)
    t4 = p.op("div", [t3, b], dtype)
    t5 = p.op("relu", [t4], dtype)
    t6 = p.op("threshold_backward", [t2, a], dtype, threshold=0.0)
    t7 = p.op("pow", [t6, 2.0], "f32")
    t8 = p.op("neg", [t7], dtype)
    p.output(t5)
    p.output(t8)
    p.output(p.op("cast", [t3], "bf16"))
    ins = [synth.random_tensor(rng, shape, dtype), synth.random_tensor(rng, shape, dtype),
           synth.random_tensor(rng, shape[-1:], dtype)]
    want = oracle_mod.run(p.text(), ins)
    got, _ = parity.gpu_run(p, ins)
    for g, w, s in zip(got, want, p.outputs):
        parity.assert_bitexact(g, w, s.dtype, s.buf)


def test_pointwise_special_values(oracle_mod):
    say("pointwise special values")
    vals = np.array([-0.0, 0.0, np.nan, np.inf, -np.inf, 1e-40, -1e-40, 3.0e38, -2.5, 65520.0, 1.0 + 2 ** -8,
                     2.0 ** -25, 6e-5, -7e-6, 1.0, -1.0], np.float32)
    p = Program()
    x = p.input("x", "f32", (16,))
    y = p.input("y", "f32", (16,))
    p.output(p.op("relu", [x], "f32"))
    p.output(p.op("threshold_backward", [y, x], "f32", threshold=0.0))
    p.output(p.op("cast", [x], "bf16"))
    p.output(p.op("cast", [x], "f16"))
    p.output(p.op("div", [y, x], "f32"))
    p.output(p.op("mul", [x, x], "bf16"))
    p.output(p.op("add", [x, y], "f16", alpha=3.0))
    ins = [vals, vals[::-1].copy()]
    want = oracle_mod.run(p.text(), ins)
    got, _ = parity.gpu_run(p, ins)
    for g, w, s in zip(got, want, p.outputs):
        parity.assert_bitexact(g, w, s.dtype, s.buf)


def _cast_patterns() -> np.ndarray:
    """fp32 bit patterns around every rounding decision of bf16 and fp16: all
    exponents, mantissas at and next to the halfway points (both parities of
    the kept bit), subnormals, zeros, infinities and NaNs."""
    exps = np.arange(256, dtype=np.uint32) << 23
    lows = []
    for keep in (16, 13):  # bf16 keeps the top 16 bits; fp16 rounds at mantissa bit 13 (normal range)
        half = 1 << (keep - 1)
        for hi in (0, 1, 2, 3, 0x3FF, 0x7F):  # kept-bit parities and saturating mantissas
            base = (hi << keep) & 0x7FFFFF
            for d in (-1, 0, 1):
                lows.append((base + half + d) & 0x7FFFFF)
        lows += [0, 0x7FFFFF, 1]
    low = np.array(lows, np.uint32)
    bits = (exps[:, None] | low[None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    # fp16 subnormal range: exponents 102..112 with dense mantissas
    rng = np.random.default_rng(7)
    sub = (rng.integers(102, 113, 4096).astype(np.uint32) << 23) | rng.integers(0, 1 << 23, 4096).astype(np.uint32)
    bits = np.concatenate([bits, sub, np.array([0x7FC00001, 0xFF800000, 0x7F800000, 0x7F7FFFFF, 0x477FF000,
                                                0x477FEFFF, 0x33000000, 0x33000001], np.uint32)])
    return bits.view(np.float32)


def test_cast_rounding_bit_patterns(oracle_mod):
    say("cast rounding bit patterns")
    x = _cast_patterns()
    p = Program()
    xi = p.input("x", "f32", x.shape)
    p.output(p.op("cast", [xi], "bf16"))
    p.output(p.op("cast", [xi], "f16"))
    p.output(p.op("relu", [xi], "bf16"))
    want = oracle_mod.run(p.text(), [x])
    got, _ = parity.gpu_run(p, [x])
    for g, w, s in zip(got, want, p.outputs):
        parity.assert_bitexact(g, w, s.dtype, s.buf)


def test_views_broadcast_and_output_copies(oracle_mod):
    say("views / broadcast / copies")
    rng = np.random.default_rng(3)
    p = Program()
    m = p.input("m", "f32", (33, 40))
    c = p.input("c", "f32", (33, 1))
    s = p.op("add", [m.T, 1.0], "f32", shape=(40, 33))
    q = p.op("mul", [m, c], "bf16")
    p.output(s)
    p.output(q)
    p.outputs.append(programs.Spec(q.buf, "f32", (40, 33), (1, 40), 0))  # transposed view, widened
    p.outputs.append(programs.Spec(m.buf, "f16", (33, 20), (40, 2), 1))  # strided input view
    p.output(p.op("full", [], "f16", shape=(5, 3), value=-1.25))
    ins = [synth.random_tensor(rng, (33, 40), "f32"), synth.random_tensor(rng, (33, 1), "f32")]
    want = oracle_mod.run(p.text(), ins)
    got, _ = parity.gpu_run(p, ins)
    for g, w, sp in zip(got, want, p.outputs):
        parity.assert_bitexact(g, w, sp.dtype, sp.buf)


# ----------------------------------------------------------- reductions --

@pytest.mark.parametrize("shape,dims,op", [
    ((64, 10), [0], "sum"), ((256, 1024), [0], "sum"), ((1000, 37), [0], "sum"),
    ((640,), None, "mean"), ((300000,), None, "sum"), ((512, 2048), None, "mean"),
    ((7, 9, 11), [1], "sum"), ((6, 5, 4), [-1, 0], "mean"), ((0, 4), [0], "sum"), ((129, 3), [1], "sum"),
    # few outputs over many partials: the combine runs a workgroup per output
    ((4, 300000), [1], "sum"), ((100000, 8), [0], "mean")])
def test_reductions(oracle_mod, shape, dims, op):
    say("reduction", shape, dims, op)
    rng = np.random.default_rng(5)
    p = Program()
    x = p.input("x", "f32", shape)
    nd = len(shape)
    red = set(range(nd)) if dims is None else {d % nd for d in dims}
    out_shape = tuple(s for i, s in enumerate(shape) if i not in red)
    sq = p.op("pow", [x, 2.0], "f32")
    r = p.op(op, [sq], "f32", out_shape, dims=dims)
    p.output(r)
    p.output(p.op(op, [x], "bf16", out_shape, dims=dims))
    ins = [synth.random_tensor(rng, shape, "f32")]
    got, _ = parity.gpu_run(p, ins)
    want = oracle_mod.run(p.text(), ins)
    vals = {"x": ins[0], sq.buf: want[0] * 0}  # placeholder, replaced below
    sqv = (ins[0].astype(np.float32) * ins[0].astype(np.float32)).astype(np.float32)
    vals[sq.buf] = sqv
    for j, (g, w) in enumerate(zip(got, want)):
        opj = p.ops[1] if j == 0 else p.ops[2]
        exact, mag = parity.reduction_reference(opj, vals)
        parity.assert_contraction(g.reshape(out_shape), w.reshape(out_shape), exact, mag, opj.out.dtype, opj.name)


# --------------------------------------------------------- contractions --

def _mm_case(oracle_mod, m, k, n, dtype, ta=False, tb=False, bias=True, seed=0, chain=False, **opts):
    rng = np.random.default_rng(seed)
    p = Program()
    A = p.input("A", dtype, (k, m) if ta else (m, k))
    B = p.input("B", dtype, (n, k) if tb else (k, n))
    av = A.T if ta else A
    bv = B.T if tb else B
    if bias:
        bi = p.input("bias", dtype, (n,))
        y = p.op("addmm", [bi, av, bv], dtype, (m, n), alpha=1.0, beta=1.0)
    else:
        y = p.op("mm", [av, bv], dtype, (m, n))
    if chain:
        z = p.op("relu", [y], dtype)
        p.output(z)
    else:
        p.output(y)
    ins = [synth.random_tensor(rng, (k, m) if ta else (m, k), dtype),
           synth.random_tensor(rng, (n, k) if tb else (k, n), dtype)]
    if bias:
        ins.append(synth.random_tensor(rng, (n,), dtype))
    got, prog = parity.gpu_run(p, ins, **opts)
    want = oracle_mod.run(p.text(), ins)
    vals = {"A": ins[0], "B": ins[1]}
    if bias:
        vals["bias"] = ins[2]
    exact, mag = parity.contraction_reference(p.ops[0], vals, None)
    if chain:
        exact = np.maximum(exact, 0)
    parity.assert_contraction(got[0], want[0], exact, mag, dtype, f"mm {m}x{k}x{n} {dtype} ta={ta} tb={tb}")
    return got, want, prog


@pytest.mark.parametrize("m,k,n", [(64, 128, 256), (64, 256, 10), (5, 7, 3), (130, 70, 65)])
@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True)])
def test_fp32_contraction_bitexact(oracle_mod, m, k, n, ta, tb):
    """The fp32 tile accumulates each output sequentially in k with fma, the
    oracle's definition, so results agree bit for bit."""
    say("fp32 mm", m, k, n, ta, tb)
    got, want, _ = _mm_case(oracle_mod, m, k, n, "f32", ta, tb, seed=m + k + n)
    parity.assert_bitexact(got[0], want[0], "f32", "fp32 mm")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("m,k,n,ta,tb", [
    (256, 512, 1024, False, False), (200, 136, 72, False, False), (64, 64, 64, True, False),
    (1024, 256, 64, True, False), (256, 64, 1024, False, True), (130, 100, 250, True, True),
    (33, 520, 17, False, False)])
def test_mfma_contraction(oracle_mod, dtype, m, k, n, ta, tb):
    say("mfma mm", dtype, m, k, n, ta, tb)
    _mm_case(oracle_mod, m, k, n, dtype, ta, tb, seed=m * 7 + n, chain=(m % 2 == 0))


@pytest.mark.parametrize("split", [2, 4])
def test_mfma_split_k(oracle_mod, split):
    say("mfma split-K", split)
    _mm_case(oracle_mod, 192, 1024, 320, "bf16", False, False, seed=split, gemm_split_k=split)


@pytest.mark.parametrize("m,k,n", [(1, 4096, 64), (1, 96, 40), (1, 1000, 24), (1, 64, 7),
                                   # multi-row slabs (decode-shaped): full, ragged and several slabs
                                   (2, 4096, 48), (3, 1000, 24), (4, 512, 40), (5, 96, 7), (8, 4096, 64),
                                   (6, 2048, 37)])
def test_gemv_q8(oracle_mod, m, k, n):
    say("gemv q8", m, k, n)
    rng = np.random.default_rng(k + n + m)
    nb = (k + 31) // 32
    p = Program()
    x = p.input("x", "bf16", (m, k))
    q = p.input("q", "i8", (n, k))
    s = p.input("s", "f32", (n, nb))
    b = p.input("b", "f32", (n,))
    z = p.op("addmm_q8", [b, x, q, s], "bf16", (m, n))
    p.output(p.op("relu", [z], "bf16"))
    ins = [synth.random_tensor(rng, (m, k), "bf16"), synth.random_tensor(rng, (n, k), "i8"),
           (0.01 * (1 - rng.random((n, nb)))).astype(np.float32), synth.random_tensor(rng, (n,), "f32", 0.3)]
    got, _ = parity.gpu_run(p, ins)
    want = oracle_mod.run(p.text(), ins)
    exact, mag = parity.contraction_reference(p.ops[0], dict(zip(["x", "q", "s", "b"], ins)), None)
    parity.assert_contraction(got[0], want[0], np.maximum(exact, 0), mag, "bf16", "gemv q8")


@pytest.mark.parametrize("m,k,xdt", [(1, 4096, "bf16"), (1, 96, "bf16"), (1, 1000, "bf16"), (1, 200, "f32"),
                                     (3, 1000, "bf16"), (5, 256, "f16"), (4, 4096, "bf16")])
def test_gemv_xq_codes_bitexact(oracle_mod, m, k, xdt):
    """One-hot weights (n = k, scales 1) return fl(d * code) per activation
    element: the quantised codes and block scales equal the oracle's bit for
    bit (ragged K, the register and LDS activation paths, several slabs)."""
    say("gemv xq codes", m, k, xdt)
    rng = np.random.default_rng(k + m)
    nb = (k + 31) // 32
    p = Program()
    x = p.input("x", xdt, (m, k))
    q = p.input("q", "i8", (k, k))
    s = p.input("s", "f32", (k, nb))
    p.output(p.op("mm_q8", [x, q, s], "f32", (m, k), xq=1.0))
    xv = synth.random_tensor(rng, (m, k), xdt, 2.0)
    if k >= 64:
        xv.reshape(-1)[:32] = 0  # an all-zero block (d = 0) in row 0
    ins = [xv, np.eye(k, dtype=np.int8), np.ones((k, nb), np.float32)]
    got, _ = parity.gpu_run(p, ins)
    (want,) = oracle_mod.run(p.text(), ins)
    parity.assert_bitexact(got[0], want, "f32", "xq codes")


@pytest.mark.parametrize("m,k,n", [(1, 4096, 64), (1, 1000, 24), (2, 4096, 48), (6, 2048, 37), (4, 96, 7)])
def test_gemv_xq(oracle_mod, m, k, n):
    say("gemv xq", m, k, n)
    rng = np.random.default_rng(k + n + m + 1)
    nb = (k + 31) // 32
    p = Program()
    x = p.input("x", "bf16", (m, k))
    q = p.input("q", "i8", (n, k))
    s = p.input("s", "f32", (n, nb))
    b = p.input("b", "f32", (n,))
    z = p.op("addmm_q8", [b, x, q, s], "bf16", (m, n), xq=1.0)
    p.output(p.op("relu", [z], "bf16"))
    ins = [synth.random_tensor(rng, (m, k), "bf16"), synth.random_tensor(rng, (n, k), "i8"),
           (0.01 * (1 - rng.random((n, nb)))).astype(np.float32), synth.random_tensor(rng, (n,), "f32", 0.3)]
    got, _ = parity.gpu_run(p, ins)
    want = oracle_mod.run(p.text(), ins)
    exact, mag = parity.contraction_reference(p.ops[0], dict(zip(["x", "q", "s", "b"], ins)), None)
    parity.assert_contraction(got[0], want[0], np.maximum(exact, 0), mag, "bf16", "gemv xq")


def _gemv_chain(m, k, n, xq, slots):
    """An int8 GEMV whose whole pointwise chain fuses into its epilogue:
    broadcast and full-shape view operands, scalars, alpha forms, rev
    division, square, sqrt, neg, relu, mixed dtypes, and (slots=True) a value
    saved and reused by threshold_backward."""
    nb = (k + 31) // 32
    p = Program()
    x = p.input("x", "bf16", (m, k))
    q = p.input("q", "i8", (n, k))
    s = p.input("s", "f32", (n, nb))
    b = p.input("b", "f32", (n,))
    c = p.input("c", "bf16", (n,))
    T = p.input("T", "f32", (m, n))
    b2 = p.input("b2", "f16", (n,))
    z = p.op("addmm_q8", [b, x, q, s], "bf16", (m, n), **({"xq": 1.0} if xq else {}))
    u = p.op("sub", [z, c], "bf16", alpha=0.75)
    v = p.op("mul", [u, 1.5], "f32")
    if slots:
        w = p.op("div", [T, v], "f32")
        y = p.op("threshold_backward", [w, u], "bf16", threshold=0.125)
    else:
        w = p.op("div", [v, T], "f32")
        w2 = p.op("pow", [w], "f16", exponent=2.0)
        w3 = p.op("sqrt", [w2], "f32")
        w4 = p.op("neg", [w3], "bf16")
        w5 = p.op("add", [w4, b2], "f32", alpha=2.0)
        y = p.op("relu", [w5], "f16")
    p.output(y)
    rng = np.random.default_rng(m * 7 + k + n)
    ins = [synth.random_tensor(rng, (m, k), "bf16"), synth.random_tensor(rng, (n, k), "i8"),
           (0.01 * (1 - rng.random((n, nb)))).astype(np.float32), synth.random_tensor(rng, (n,), "f32", 0.3),
           synth.random_tensor(rng, (n,), "bf16", 0.5), synth.random_tensor(rng, (m, n), "f32", 2.0),
           synth.random_tensor(rng, (n,), "f16", 0.5)]
    return p, ins


@pytest.mark.parametrize("m,k,n,xq,slots", [(1, 1024, 40, False, False), (3, 256, 40, False, True),
                                           (6, 512, 37, True, False), (1, 4096, 64, True, True)])
def test_gemv_epilogue_chain(oracle_mod, m, k, n, xq, slots):
    """The GEMV epilogue evaluates a fused chain element by element; with
    epilogue fusion off the chain runs as elementwise tasks through the
    expression machine.  Both agree bit for bit, and every node of the probe
    (which fuses the chain too, storing each value) matches the oracle."""
    say("gemv epilogue chain", m, k, n, xq, slots)
    base, ins = _gemv_chain(m, k, n, xq, slots)
    o1, p1 = parity.gpu_run(base, [a.copy() for a in ins])
    assert "+side" in p1.dump() and p1.query()["n_stages"] == 1
    o2, p2 = parity.gpu_run(base, [a.copy() for a in ins], fuse_epilogues=0)
    assert p2.query()["n_stages"] > 1
    parity.assert_bitexact(o1[0], o2[0], base.outputs[0].dtype, "chain output")
    probe = base.probe()
    o3, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(base, probe, o3)
    assert parity.check_per_node(oracle_mod, base, ins, vals) == len(base.ops)


def test_gemv_several_items_per_workgroup():
    """A 3-layer int8 stack on a 24-workgroup grid (each workgroup takes
    several items of a layer, in sequence): the outputs equal those of the
    default grid (one item per workgroup) bit for bit."""
    say("gemv on a 24-workgroup grid vs the default grid")
    cfg = dict(kind="gemv", k=1024, n=1024, layers=3)
    prog = programs.build(cfg)
    ins = programs.inputs_for(cfg, 4)
    a, pa = parity.gpu_run(prog, [x.copy() for x in ins])
    b, pb = parity.gpu_run(prog, [x.copy() for x in ins], force_grid=24)
    assert pb.query()["grid_size"] == 24 and pa.query()["grid_size"] > 24
    for x, y, sp in zip(a, b, prog.outputs):
        parity.assert_bitexact(y, x, sp.dtype, sp.buf)


# ------------------------------------------------------------ whole steps --

SMALL = {
    "c1": dict(programs.CONFIGS["c1"]),
    "c2s": dict(kind="mlp", dims=(192, 320, 256, 48), batch=96, dtype="bf16", lr=1e-3),
    "c3s": dict(kind="gemv", k=1024, n=1024, layers=3),
    "c3r": dict(kind="gemv", k=1024, n=1024, layers=3, rows=6),  # decode rows in two slabs
    # activations quantised to Q8_0 inside each product
    "c3q": dict(kind="gemv", k=1024, n=1024, layers=3, xq=True),
    "c3qr": dict(kind="gemv", k=1024, n=1024, layers=3, rows=6, xq=True),
    "c4s": dict(kind="mlp", dims=(256, 384, 256, 128), batch=160, dtype="bf16", lr=1e-4),
    "c5s": dict(kind="residual", width=256, layers=4, batch=96, dtype="f16", lr=1e-4),
    # AdamW in place of SGD: two float32 states per parameter, updated in place
    "c1a": dict(programs.CONFIGS["c1"], optimizer=programs.AdamW()),
    "c2sa": dict(kind="mlp", dims=(192, 320, 256, 48), batch=96, dtype="bf16", lr=1e-3,
                 optimizer=programs.AdamW(), adam_t=5),
    "c5sa": dict(kind="residual", width=256, layers=4, batch=96, dtype="f16", lr=1e-4,
                 optimizer=programs.AdamW(weight_decay=0.1), adam_t=2),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_whole_step_per_node(oracle_mod, name):
    cfg = SMALL[name]
    say("whole step per node", name)
    base = programs.build(cfg)
    probe = base.probe()
    ins = programs.inputs_for(cfg, 0)
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(base, probe, outs)
    n = parity.check_per_node(oracle_mod, base, ins, vals)
    assert n == len(base.ops)


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_equals_unfused(name):
    """The fused schedule and the probe (everything materialised) agree bitwise
    on the shared outputs."""
    cfg = SMALL[name]
    say("fused == probe", name)
    base = programs.build(cfg)
    probe = base.probe()
    ins = programs.inputs_for(cfg, 1)
    o1, p1 = parity.gpu_run(base, [a.copy() for a in ins])
    o2, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    assert p1.query()["n_stages"] >= 1
    for a, b, s in zip(o1, o2, base.outputs):
        parity.assert_bitexact(a, b, s.dtype, s.buf)


def _column_sum_values(dump: str) -> set:
    """Values a column reduction writes, run as its own task or inside a
    contraction ("+column sums of B:"): its root and its side values."""
    names = set()
    for line in dump.splitlines():
        line = line.strip()
        if line.startswith("reduce_cols") or line.startswith("reduce_final"):
            rest = line.split(" : ", 1)[1]
        elif "+column sums of B: " in line:
            rest = line.split("+column sums of B: ", 1)[1]
        else:
            continue
        names.add(rest.split(" ", 1)[0])
        if "+side" in rest:
            side = rest.split("+side", 1)[1].split("(")[0].split("[")[0]
            names.update(side.split())
    return names


def _assert_sums_within_one_ulp(got, want, spec):
    """Column-sum values added in another row order: one ulp apart at most."""
    g, w = parity.f32_of(got, spec.dtype), parity.f32_of(want, spec.dtype)
    if spec.dtype == "f32":
        tol = np.spacing(np.abs(w).astype(np.float32))
    else:
        tol = parity.ulp16(w, spec.dtype)
    assert np.all(np.abs(g - w) <= tol), f"{spec.buf}: more than one ulp apart"


@pytest.mark.parametrize("name", ["c1", "c2s", "c4s", "c5s", "c2sa"])
def test_register_epilogue_matches_batches(name):
    """Contraction epilogues run from registers (the default where the
    scheduler marks them) give the same bits as the expression machine's
    batches (batch_epilogues=1) on every output that no column sum feeds.  A
    column sum run by a weight-gradient tile or read straight from memory by
    32 row lanes adds its rows in another order than the batches, so the
    values it writes (the bias gradients and their updates) agree within one
    unit in the last place instead (both are checked against the oracle per
    node elsewhere)."""
    cfg = SMALL[name]
    say("register epilogue == batches", name)
    base = programs.build(cfg)
    ins = programs.inputs_for(cfg, 3)
    o1, p1 = parity.gpu_run(base, [a.copy() for a in ins])
    o2, _ = parity.gpu_run(base, [a.copy() for a in ins], batch_epilogues=1)
    d1 = p1.dump()
    assert "[register epilogue]" in d1
    assert "[rows summed directly]" in d1 or "+column sums of B: " in d1
    summed = _column_sum_values(d1)
    for a, b, s in zip(o1, o2, base.outputs):
        if s.buf not in summed:
            parity.assert_bitexact(a, b, s.dtype, s.buf)
        else:
            _assert_sums_within_one_ulp(a, b, s)


# Bias gradients summed by the first tile row of their weight-gradient
# product (colsum_fusion=1 forces it where the default would not).  A batch
# of 128 or 192 rows puts K on whole 64-deep slices, so the sums come out of
# the product's main loop (an even and an odd number of slices); the 160 and
# 96 rows of the small configs do not, and their tiles read the rows again
# after the product; 48 output columns leave a partial tile.
COLSUM = {
    "mlp-bf16-k128": dict(kind="mlp", dims=(256, 384, 256, 128), batch=128, dtype="bf16", lr=1e-4),
    "res-f16-k192": dict(kind="residual", width=256, layers=4, batch=192, dtype="f16", lr=1e-4),
    "c4s": SMALL["c4s"],
    "c2s": SMALL["c2s"],
    # AdamW: the tile's epilogue runs on the batches, the sums after them
    "c5sa": SMALL["c5sa"],
}


@pytest.mark.parametrize("tile", [1, 2])
@pytest.mark.parametrize("name", list(COLSUM))
def test_column_sums_in_weight_gradient_tiles(oracle_mod, name, tile):
    """Per node against the oracle with the sums in the tiles (128x128 and
    64x64 tiles; the probe schedule, which fuses them too except with AdamW),
    and against the same step with the sums run as reductions of their own:
    bit-identical except the summed values (one ulp)."""
    cfg = COLSUM[name]
    say("column sums in weight-gradient tiles", name, "tile", tile)
    base = programs.build(cfg)
    probe = base.probe()
    ins = programs.inputs_for(cfg, 4)
    outs, pp = parity.gpu_run(probe, [a.copy() for a in ins], colsum_fusion=1, gemm_tile=tile)
    # (AdamW's probe returns values that read the sums, which keeps them
    # reductions there; its fused step is checked against the unfused one)
    assert ("+column sums of B: " in pp.dump()) == (name != "c5sa")
    vals = parity.probe_values(base, probe, outs)
    assert parity.check_per_node(oracle_mod, base, ins, vals) == len(base.ops)
    o1, p1 = parity.gpu_run(base, [a.copy() for a in ins], colsum_fusion=1, gemm_tile=tile)
    o2, p2 = parity.gpu_run(base, [a.copy() for a in ins], colsum_fusion=-1, gemm_tile=tile)
    d1 = p1.dump()
    assert "+column sums of B: " in d1 and "+column sums of B: " not in p2.dump()
    summed = _column_sum_values(d1)
    for a, b, s in zip(o1, o2, base.outputs):
        if s.buf not in summed:
            parity.assert_bitexact(a, b, s.dtype, s.buf)
        else:
            _assert_sums_within_one_ulp(a, b, s)


@pytest.mark.parametrize("name", ["c2s", "c5s"])
def test_ordinary_launch_matches_cooperative(name):
    """launch_mode=1 (ordinary launch of the co-resident grid) runs the same
    kernel on the same plan: outputs are bit-identical to the cooperative
    launch, and no barrier aborts."""
    cfg = SMALL[name]
    say("launch modes", name)
    base = programs.build(cfg)
    ins = programs.inputs_for(cfg, 2)
    o1, _ = parity.gpu_run(base, [a.copy() for a in ins], launch_mode=0)
    o2, p2 = parity.gpu_run(base, [a.copy() for a in ins], launch_mode=1)
    for a, b, s in zip(o1, o2, base.outputs):
        parity.assert_bitexact(a, b, s.dtype, s.buf)


def test_graph_replay_matches_eager_steps():
    """Four steps over four resident batches, captured once and replayed three
    times with eager work and synchronisations in between, give after every
    replay exactly the parameters and loss of the same twelve steps run
    eagerly (state feedback through the in-place updates)."""
    import torch
    from persistent_whole_step_amd import tk
    cfg = SMALL["c2s"]
    say("graph replay c2s")
    prog = programs.build(cfg)
    p = tk.compile(prog.text(), device=0, launch_mode=1)
    base = programs.inputs_for(cfg, 3)
    batches = [programs.inputs_for(cfg, 10 + j)[:2] for j in range(4)]

    def state():
        params = [parity.to_torch(a, s.dtype) for a, s in zip(base[2:], prog.inputs[2:])]
        xs = [[parity.to_torch(b[0], prog.inputs[0].dtype), parity.to_torch(b[1], prog.inputs[1].dtype)]
              for b in batches]
        bufs = p.allocate(*(xs[0] + params))
        variants = [(x + params, tk.ExecutionBuffers(
            tuple(params[p._inplace_map()[s] - 2] if s in p._inplace_map() else o
                  for s, o in enumerate(bufs.outputs)), bufs.workspace)) for x in xs]
        return params, variants

    e_params, e_vars = state()
    g_params, g_vars = state()
    graph = tk.StepGraph(p, g_vars)
    junk = torch.zeros(1 << 20, device="cuda:0")
    for rep in range(3):
        for ins, bufs in e_vars:
            p.run_into(*ins, buffers=bufs)
        graph.replay()
        junk.add_(1.0)  # eager work of the program's own between replays
        torch.cuda.synchronize()
        for a, b, s in zip(e_params, g_params, prog.inputs[2:]):
            parity.assert_bitexact(parity.to_numpy(b, s.dtype), parity.to_numpy(a, s.dtype), s.dtype, s.buf)
        le = parity.to_numpy(e_vars[-1][1].outputs[0], prog.outputs[0].dtype)
        lg = parity.to_numpy(g_vars[-1][1].outputs[0], prog.outputs[0].dtype)
        parity.assert_bitexact(lg, le, prog.outputs[0].dtype, "loss")
    aborted, _ = p.workspace_status(g_vars[0][1].workspace)
    assert not aborted


def _staged_program(kind: str, dt: str, n: int) -> Program:
    """Programs whose in-place update cannot be written where it is computed,
    so the scheduler stages it and commits it after the last read of the
    target (the codegen page's final commit stage):
      tile_reads: the update's gradient tile reads the target itself;
      after_store: an op of the same tile reads the target after the update;
      pointwise: a later pointwise op reads the target."""
    p = Program()
    a = p.input("a", dt, (n, n))
    W = p.input("W", dt, (n, n))
    if kind == "tile_reads":
        g = p.op("mm", [a, W], dt, (n, n))
        p.output(p.op("sub", [W, g], dt, alpha=0.5), inplace_of=W)
        p.output(g)
    elif kind == "after_store":
        b = p.input("b", dt, (n, n))
        g = p.op("mm", [a, b], dt, (n, n))
        wn = p.op("sub", [W, g], dt, alpha=0.5)
        p.output(p.op("mul", [W, g], dt))
        p.output(wn, inplace_of=W)
    else:
        wn = p.op("sub", [W, a], dt, alpha=0.5)
        p.output(wn, inplace_of=W)
        p.output(p.op("mul", [W, 2.0], dt))
    return p


@pytest.mark.parametrize("kind", ["tile_reads", "after_store", "pointwise"])
@pytest.mark.parametrize("dt,n", [("bf16", 192), ("bf16", 520), ("f32", 130)])
def test_staged_commit(oracle_mod, kind, dt, n):
    """Staged (transactional) in-place commits on the GPU: the plan stages the
    update; every op, checked per node against the oracle from the original
    inputs, saw the target's old value; the fused run leaves the same bits in
    the caller's target tensor as the probe run."""
    say("staged commit", kind, dt, n)
    from persistent_whole_step_amd import tk
    base = _staged_program(kind, dt, n)
    probe = base.probe()
    for prog in (base, probe):
        assert tk.compile(prog.text(), device=-1).query()["staged_commits"] >= 1
    rng = np.random.default_rng(n)
    ins = [synth.random_tensor(rng, s.shape, s.dtype, 0.25) for s in base.inputs]
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(base, probe, outs)
    assert parity.check_per_node(oracle_mod, base, ins, vals) == len(base.ops)
    fused, p = parity.gpu_run(base, [a.copy() for a in ins])
    assert p.query()["staged_commits"] >= 1
    for a, b, s in zip(fused, outs, base.outputs):
        parity.assert_bitexact(a, b, s.dtype, s.buf)


def test_graph_replayed_probe_steps_per_node(oracle_mod):
    """A captured 20-step replay checked against the oracle: the probe program
    (every op's value returned) of the c2s step is captured once per resident
    batch (4 graphs, state fed back through the in-place updates) and the
    graphs are replayed in rotation for 20 steps; after each step every op is
    checked per node against the oracle on that step's batch and on the
    parameters the previous replay left."""
    import torch
    from persistent_whole_step_amd import tk
    cfg = SMALL["c2s"]
    say("graph-replayed probe, 20 steps, c2s")
    base = programs.build(cfg)
    probe = base.probe()
    p = tk.compile(probe.text(), device=0, launch_mode=1)
    start = programs.inputs_for(cfg, 4)
    batches = [programs.inputs_for(cfg, 20 + j)[:2] for j in range(4)]
    params = [parity.to_torch(a, s.dtype) for a, s in zip(start[2:], probe.inputs[2:])]
    xs = [[parity.to_torch(b[0], probe.inputs[0].dtype), parity.to_torch(b[1], probe.inputs[1].dtype)]
          for b in batches]
    bufs = p.allocate(*(xs[0] + params))
    graphs = [tk.StepGraph(p, [(x + params, bufs)]) for x in xs]
    state = [a.copy() for a in start[2:]]
    for step in range(20):
        j = step % 4
        graphs[j].replay()
        torch.cuda.synchronize()
        outs = [parity.to_numpy(o, sp.dtype) for o, sp in zip(bufs.outputs, probe.outputs)]
        vals = parity.probe_values(base, probe, outs)
        ins = [batches[j][0], batches[j][1]] + state
        assert parity.check_per_node(oracle_mod, base, ins, vals) == len(base.ops), step
        state = [parity.to_numpy(t, sp.dtype) for t, sp in zip(params, probe.inputs[2:])]
    p.check_workspace(bufs.workspace)


def test_compiled_step_capture_restores_state_and_replays():
    """CompiledTrainingStep.capture: warmup and capture leave the supplied
    state as it was; each replay advances it exactly as the eager compiled
    step does from the same state, for 20 steps (the eager step's program is
    checked per node against the oracle in test_compile_training_step)."""
    import torch
    from persistent_whole_step_amd import frontend
    from .test_frontend import mlp_step
    say("capture API, 20 replays")
    gen = torch.Generator().manual_seed(9)
    shapes = {"W1": (96, 160), "b1": (160,), "W2": (160, 48), "b2": (48,)}
    params = {k: (torch.randn(*s, generator=gen) / 6).to(torch.bfloat16) for k, s in shapes.items()}
    x = torch.randn(40, 96, generator=gen).to(torch.bfloat16).cuda()
    t = torch.randn(40, 48, generator=gen).to(torch.bfloat16).cuda()
    step = frontend.compile_training(mlp_step, (params, x.cpu(), t.cpu()))
    pg = {k: v.cuda() for k, v in params.items()}
    pe = {k: v.cuda() for k, v in params.items()}
    cap = step.capture(pg, x, t, warmup=3)
    for k in pg:
        assert torch.equal(pg[k].view(torch.int16), pe[k].view(torch.int16)), k
    for i in range(20):
        loss_g, new_g = cap.replay()
        loss_e, new_e = step(pe, x, t)
        torch.cuda.synchronize()
        assert torch.equal(loss_g.view(torch.int16), loss_e.view(torch.int16)), i
        for k in pg:
            assert new_g[k].data_ptr() == pg[k].data_ptr()
            assert torch.equal(pg[k].view(torch.int16), pe[k].view(torch.int16)), (i, k)


@pytest.mark.parametrize("name", ["c2s", "c5s", "c2sa", "c3s"])
def test_race_modes_bit_identical(name):
    """The schedule's race-exposing run modes give the default run's bits:
    every workgroup sleeping a seeded pseudo-random time before each work
    item (stagger), the workspace filled with a NaN byte pattern before the
    launch (poison: no value is read before it is written), and one op per
    stage (barrier_every_op)."""
    import torch
    from persistent_whole_step_amd import tk
    cfg = SMALL[name]
    say("race modes", name)
    base = programs.build(cfg)
    ins = programs.inputs_for(cfg, 5)
    ref, _ = parity.gpu_run(base, [a.copy() for a in ins], launch_mode=1)

    def run(poison=False, stagger=0, **opts):
        p = tk.compile(base.text(), device=0, launch_mode=1, **opts)
        tins = [parity.to_torch(a.copy(), sp.dtype) for a, sp in zip(ins, base.inputs)]
        bufs = p.allocate(*tins)
        if poison:
            # the header keeps its barrier state; the arena gets NaN bytes
            hdr = int(re.search(r"workspace: (\d+) header", p.dump()).group(1))
            bufs.workspace[hdr:].fill_(0xFF)
            for o, sp in zip(bufs.outputs, base.outputs):
                if not any(o.data_ptr() == t.data_ptr() for t in tins):
                    o.reshape(-1).view(torch.uint8).fill_(0xFF)
        p.set_debug(stagger_seed=stagger)
        p.run_into(*tins, buffers=bufs)
        p.check_workspace(bufs.workspace)
        return [parity.to_numpy(o, sp.dtype) for o, sp in zip(bufs.outputs, base.outputs)]

    for mode in (dict(stagger=0x5eed), dict(stagger=77), dict(poison=True), dict(barrier_every_op=1),
                 dict(poison=True, stagger=3, barrier_every_op=1)):
        got = run(**mode)
        for g, r, sp in zip(got, ref, base.outputs):
            parity.assert_bitexact(g, r, sp.dtype, f"{sp.buf} under {mode}")


def test_barrier_timeout_reports_aborted():
    """A grid barrier that times out (forced from the host with a one-tick
    wait limit; every workgroup still leaves the kernel) marks the workspace
    aborted: the status reads it back, the next run_into fails with
    TK_E_ABORTED before launching, and after tk_workspace_init the program
    runs again and gives a clean run's bits."""
    from persistent_whole_step_amd import tk
    cfg = SMALL["c2s"]
    say("barrier timeout -> TK_E_ABORTED")
    base = programs.build(cfg)
    ins = programs.inputs_for(cfg, 6)
    ref, _ = parity.gpu_run(base, [a.copy() for a in ins], launch_mode=1)
    p = tk.compile(base.text(), device=0, launch_mode=1)
    tins = [parity.to_torch(a.copy(), sp.dtype) for a, sp in zip(ins, base.inputs)]
    bufs = p.allocate(*tins)
    p.set_debug(deadline_ticks=1)
    p.run_into(*tins, buffers=bufs)
    aborted, stage = p.workspace_status(bufs.workspace)
    assert aborted and 0 <= stage < p.query()["n_stages"]
    with pytest.raises(tk.TkError) as e:
        p.run_into(*tins, buffers=bufs)
    assert e.value.status_name == "TK_E_ABORTED"
    with pytest.raises(tk.TkError):
        p.check_workspace(bufs.workspace)
    p.set_debug(deadline_ticks=0)
    p.init_workspace(bufs.workspace)
    tins = [parity.to_torch(a.copy(), sp.dtype) for a, sp in zip(ins, base.inputs)]
    bufs = tk.ExecutionBuffers(tuple(tins[p._inplace_map()[s]] if s in p._inplace_map() else o
                                     for s, o in enumerate(bufs.outputs)), bufs.workspace)
    p.run_into(*tins, buffers=bufs)
    p.check_workspace(bufs.workspace)
    for g, r, sp in zip(bufs.outputs, ref, base.outputs):
        parity.assert_bitexact(parity.to_numpy(g, sp.dtype), r, sp.dtype, sp.buf)


def test_c1_end_to_end_close_to_oracle(oracle_mod):
    cfg = SMALL["c1"]
    say("c1 end to end")
    base = programs.build(cfg)
    ins = programs.inputs_for(cfg, 2)
    got, _ = parity.gpu_run(base, [a.copy() for a in ins])
    want = oracle_mod.run(base.text(), [a.copy() for a in ins])
    for g, w, s in zip(got, want, base.outputs):
        np.testing.assert_allclose(parity.f32_of(g, s.dtype), parity.f32_of(w, s.dtype), rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------- full sizes --

FULL = {
    "c2": dict(programs.CONFIGS["c2"]),
    "c2a": dict(programs.CONFIGS["c2"], optimizer=programs.AdamW(), adam_t=10),
    "c3": dict(programs.CONFIGS["c3"]),
    "c3q": dict(programs.CONFIGS["c3"], xq=True),
    "c3r4": dict(programs.CONFIGS["c3"], rows=4),
    "c4": dict(programs.CONFIGS["c4"]),
    "c5": dict(programs.CONFIGS["c5"]),
}


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_per_node(oracle_mod, name, seed):
    """The workloads at their full sizes, in the launch configuration the
    bench times (ordinary launch of the co-resident grid), on three input
    seeds: every op checked per node with teacher forcing (pointwise ops and
    reductions whole, each contraction on a block of outputs with at least
    one in every 64x64 output tile, plus the edges, each computed by the
    oracle), then the bench's fused schedule equal to the probe schedule bit
    for bit on the step's outputs."""
    cfg = FULL[name]
    say("full size, sampled per node", name, "seed", seed)
    base = programs.build(cfg)
    probe = base.probe()
    ins = programs.inputs_for(cfg, seed)
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins], launch_mode=1)
    vals = parity.probe_values(base, probe, outs)
    n = parity.check_per_node_sampled(oracle_mod, base, ins, vals, seed=len(name) + 10 * seed)
    assert n == len(base.ops)
    fused, _ = parity.gpu_run(base, [a.copy() for a in ins], launch_mode=1)
    for a, b, s in zip(fused, outs, base.outputs):
        parity.assert_bitexact(a, b, s.dtype, s.buf)


# ------------------------------------------------- fast paths' fallbacks --

def _misaligned_copy(t):
    """A copy of `t` whose data pointer lies 2 bytes past a 16-byte boundary
    (a view one element into a larger buffer), with `t`'s shape and strides."""
    import torch
    big = torch.zeros(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = big[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0 and v.is_contiguous()
    return v


def test_register_epilogue_misaligned_bias_uses_batches(oracle_mod):
    """A marked tile whose bias base is not 16-byte aligned at run time runs
    its epilogue through the batches: same bits as with an aligned bias, and
    within tolerance of the oracle."""
    from persistent_whole_step_amd import tk
    say("register epilogue, misaligned bias")
    m, k, n = 192, 160, 256
    rng = np.random.default_rng(11)
    p = Program()
    A = p.input("A", "bf16", (m, k))
    B = p.input("B", "bf16", (k, n))
    bi = p.input("bias", "bf16", (n,))
    y = p.op("addmm", [bi, A, B], "bf16", (m, n), alpha=1.0, beta=1.0)
    p.output(p.op("relu", [y], "bf16"))
    ins = [synth.random_tensor(rng, (m, k), "bf16"), synth.random_tensor(rng, (k, n), "bf16"),
           synth.random_tensor(rng, (n,), "bf16")]
    prog = tk.compile(p.text(), device=0)
    assert "[register epilogue]" in prog.dump()
    tA, tB, tb = (parity.to_torch(a, s.dtype) for a, s in zip(ins, p.inputs))
    aligned = parity.to_numpy(prog(tA, tB, tb)[0], "bf16")
    shifted = parity.to_numpy(prog(tA, tB, _misaligned_copy(tb))[0], "bf16")
    parity.assert_bitexact(shifted, aligned, "bf16", "misaligned bias")
    want = oracle_mod.run(p.text(), ins)[0]
    exact, mag = parity.contraction_reference(p.ops[0], {"A": ins[0], "B": ins[1], "bias": ins[2]}, None)
    parity.assert_contraction(aligned, want, np.maximum(exact, 0), mag, "bf16", "addmm + relu")


def test_direct_column_sum_misaligned_source(oracle_mod):
    """A column sum read straight from a misaligned input takes element loads:
    same bits as from an aligned input, within tolerance of the oracle."""
    from persistent_whole_step_amd import tk
    say("direct column sum, misaligned source")
    rows, cols = 200, 512
    rng = np.random.default_rng(12)
    p = Program()
    g = p.input("g", "bf16", (rows, cols))
    p.output(p.op("sum", [g], "f32", (cols,), dims=(0,)))
    ins = [synth.random_tensor(rng, (rows, cols), "bf16")]
    prog = tk.compile(p.text(), device=0)
    assert "[rows summed directly]" in prog.dump()
    tg = parity.to_torch(ins[0], "bf16")
    aligned = parity.to_numpy(prog(tg)[0], "f32")
    shifted = parity.to_numpy(prog(_misaligned_copy(tg))[0], "f32")
    parity.assert_bitexact(shifted, aligned, "f32", "misaligned column sum")
    want = oracle_mod.run(p.text(), ins)[0]
    exact, mag = parity.reduction_reference(p.ops[0], {"g": ins[0]})
    parity.assert_contraction(aligned, want, exact, mag, "f32", "column sum")


# ------------------------------------------------------- capture front end --

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compile_training_step(oracle_mod, dtype):
    """A torch.func training step captured and compiled: its program checked
    per node against the oracle on the GPU, then the compiled step run on GPU
    tensors gives the same bits as the program, with the updated state
    written into the state tensors passed in."""
    import torch
    from persistent_whole_step_amd import frontend, tk
    from .test_frontend import mlp_step
    say("capture front end", dtype)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    gen = torch.Generator().manual_seed(5)
    shapes = {"W1": (96, 160), "b1": (160,), "W2": (160, 48), "b2": (48,)}
    params = {k: (torch.randn(*s, generator=gen) / 6).to(tdt) for k, s in shapes.items()}
    x = torch.randn(40, 96, generator=gen).to(tdt)
    t = torch.randn(40, 48, generator=gen).to(tdt)
    step = frontend.compile_training(mlp_step, (params, x, t))
    prog = step.program
    assert sorted(prog.inplace.values()) == [0, 1, 2, 3]
    from torch.utils import _pytree as pytree
    leaves, _ = pytree.tree_flatten((params, x, t))
    ins = [tk.storage_from_tensor(v, s.dtype) for v, s in zip(leaves, prog.inputs)]
    probe = prog.probe()
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(prog, probe, outs)
    assert parity.check_per_node(oracle_mod, prog, ins, vals) == len(prog.ops)
    ref, _ = parity.gpu_run(prog, [a.copy() for a in ins])
    # the fused, in-place schedule equals the oracle-checked probe run bit for bit
    for i, sp in enumerate(prog.outputs):
        parity.assert_bitexact(ref[i], outs[i], sp.dtype, f"fused vs probe {sp.buf}")
    pg = {k: v.cuda() for k, v in params.items()}
    loss, new = step(pg, x.cuda(), t.cuda())
    torch.cuda.synchronize()
    for k in pg:
        assert new[k].data_ptr() == pg[k].data_ptr()
    got, _ = pytree.tree_flatten((loss, new))  # the program's outputs, in the same order
    for g, r, s in zip(got, ref, prog.outputs):
        parity.assert_bitexact(tk.storage_from_tensor(g, s.dtype), r, s.dtype, s.buf)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compile_training_broadcast_step(oracle_mod, dtype):
    """A captured step whose gradient uses division, negation, keepdim and
    dim-wise reductions, unsqueeze and stride-0 broadcast views: per node
    against the oracle on the GPU, and the compiled step equal to the
    program run bit for bit."""
    import torch
    from persistent_whole_step_amd import frontend, tk
    from .test_frontend import misc_step
    say("capture front end, broadcast step", dtype)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    gen = torch.Generator().manual_seed(7)
    w = (torch.randn(64, 48, generator=gen) / 8).to(tdt)
    x = torch.randn(24, 64, generator=gen).to(tdt)
    t = torch.randn(24, 48, generator=gen).to(tdt)
    step = frontend.compile_training(misc_step, (w, x, t))
    prog = step.program
    assert prog.inplace == {1: 0}
    ins = [tk.storage_from_tensor(v, s.dtype) for v, s in zip((w, x, t), prog.inputs)]
    probe = prog.probe()
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(prog, probe, outs)
    assert parity.check_per_node(oracle_mod, prog, ins, vals) == len(prog.ops)
    ref, _ = parity.gpu_run(prog, [a.copy() for a in ins])
    # the fused, in-place schedule equals the oracle-checked probe run bit for bit
    for i, sp in enumerate(prog.outputs):
        parity.assert_bitexact(ref[i], outs[i], sp.dtype, f"fused vs probe {sp.buf}")
    wg = w.cuda()
    loss, w_new = step(wg, x.cuda(), t.cuda())
    torch.cuda.synchronize()
    assert w_new.data_ptr() == wg.data_ptr()
    for g, r, s in zip((loss, w_new), ref, prog.outputs):
        parity.assert_bitexact(tk.storage_from_tensor(g, s.dtype), r, s.dtype, s.buf)


def test_compile_training_adamw_step(oracle_mod):
    """AdamW written in torch and compiled: weights and both moment states
    committed in place, per node against the oracle, and equal to the
    program run bit for bit."""
    import torch
    from persistent_whole_step_amd import frontend, tk
    from .test_frontend import adamw_step, _examples
    from torch.utils import _pytree as pytree
    say("capture front end, AdamW step")
    ex = _examples("adamw", seed=3)
    step = frontend.compile_training(adamw_step, ex)
    prog = step.program
    assert prog.inplace == {1: 0, 2: 1, 3: 2}
    leaves, _ = pytree.tree_flatten(ex)
    ins = [tk.storage_from_tensor(v, s.dtype) for v, s in zip(leaves, prog.inputs)]
    probe = prog.probe()
    outs, _ = parity.gpu_run(probe, [a.copy() for a in ins])
    vals = parity.probe_values(prog, probe, outs)
    assert parity.check_per_node(oracle_mod, prog, ins, vals) == len(prog.ops)
    ref, _ = parity.gpu_run(prog, [a.copy() for a in ins])
    # the fused, in-place schedule equals the oracle-checked probe run bit for bit
    for i, sp in enumerate(prog.outputs):
        parity.assert_bitexact(ref[i], outs[i], sp.dtype, f"fused vs probe {sp.buf}")
    state = tuple(v.cuda() for v in ex[0])
    loss, new = step(state, ex[1].cuda(), ex[2].cuda())
    torch.cuda.synchronize()
    assert all(a.data_ptr() == b.data_ptr() for a, b in zip(new, state))
    got, _ = pytree.tree_flatten((loss, new))
    for g, r, s in zip(got, ref, prog.outputs):
        parity.assert_bitexact(tk.storage_from_tensor(g, s.dtype), r, s.dtype, s.buf)
