"""Whole-step programs in the ``tkir 1`` text format.

A program is the static description of one functional training step, as on
the trainkernel pages (codegen.py, the ``Program`` / ``Operation`` /
``TensorSpec`` objects used throughout ``_Generator``): named tensor views with
shape, element strides, element offset and dtype; an operation list in
topological order; the returned values; and declared in-place pairs
``{output slot -> input index}``.  The text is what both the CPU oracle and the
HIP library parse -- it is their common *input*, like the seeded tensors, and
this module computes nothing of the step itself.

Grammar (one statement per line, ``;`` starts a comment)::

    tkir 1
    in  <buf> <dtype> <shape> <strides> <offset>
    op  <name> <opcode> <outspec> <operand>* <key>=<value>*
    out <spec>
    inplace <output_slot> <input_index>
    end

``<spec>`` is ``buf:dtype:shape:strides:offset``; shapes and strides are
``x``-separated integers (``64x128``), ``-`` for rank 0.  An operand is a spec
or a scalar ``#<hexfloat>`` (the exact float32 value, written as a C99 hex
float).  Attributes: ``alpha beta threshold value exponent`` take a scalar,
``dims`` takes a ``,``-separated list or ``all``.  dtypes: f32 f16 bf16 i8.
Opcodes: add sub mul div neg relu pow threshold_backward full cast (pointwise),
mm addmm (contractions), mm_q8 addmm_q8 (contraction with an int8 weight in
32-element blocks along K and one float32 scale per block), sum mean.
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass, field

import numpy as np

POINTWISE = ("add", "sub", "mul", "div", "neg", "relu", "pow", "threshold_backward", "full", "cast")
CONTRACTIONS = ("mm", "addmm", "mm_q8", "addmm_q8")
REDUCTIONS = ("sum", "mean")


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", float(x)))[0]


def hexf(x: float) -> str:
    v = f32(x)
    if not math.isfinite(v):
        raise ValueError("non-finite scalar constants are unsupported")
    return "#" + v.hex()


def contiguous_strides(shape):
    out, acc = [], 1
    for d in reversed(shape):
        out.append(acc)
        acc *= max(1, d)
    return tuple(reversed(out))


def _dims_text(v) -> str:
    return "x".join(str(int(d)) for d in v) if len(v) else "-"


@dataclass(frozen=True)
class Spec:
    buf: str
    dtype: str
    shape: tuple
    strides: tuple
    offset: int = 0

    def text(self) -> str:
        return f"{self.buf}:{self.dtype}:{_dims_text(self.shape)}:{_dims_text(self.strides)}:{self.offset}"

    @property
    def T(self) -> "Spec":
        assert len(self.shape) == 2
        return Spec(self.buf, self.dtype, self.shape[::-1], self.strides[::-1], self.offset)

    def view(self, shape, strides, offset=0) -> "Spec":
        return Spec(self.buf, self.dtype, tuple(shape), tuple(strides), int(offset))

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


@dataclass
class Op:
    name: str
    opcode: str
    out: Spec
    operands: list
    attrs: dict = field(default_factory=dict)


class Program:
    def __init__(self):
        self.inputs: list[Spec] = []
        self.ops: list[Op] = []
        self.outputs: list[Spec] = []
        self.inplace: dict[int, int] = {}
        self._names: set[str] = set()

    # -- construction -------------------------------------------------------
    def _fresh(self, base: str) -> str:
        name, i = base, 1
        while name in self._names:
            i += 1
            name = f"{base}_{i}"
        self._names.add(name)
        return name

    def input(self, name: str, dtype: str, shape) -> Spec:
        shape = tuple(int(d) for d in shape)
        spec = Spec(self._fresh(name), dtype, shape, contiguous_strides(shape), 0)
        self.inputs.append(spec)
        return spec

    def op(self, opcode: str, operands, dtype: str, shape=None, name: str | None = None, **attrs) -> Spec:
        if shape is None:
            shape = next(o.shape for o in operands if isinstance(o, Spec))
        shape = tuple(int(d) for d in shape)
        out = Spec(self._fresh(name or opcode), dtype, shape, contiguous_strides(shape), 0)
        self.ops.append(Op(out.buf, opcode, out, list(operands), dict(attrs)))
        return out

    def output(self, spec: Spec, inplace_of: Spec | None = None) -> int:
        self.outputs.append(spec)
        slot = len(self.outputs) - 1
        if inplace_of is not None:
            self.inplace[slot] = [i.buf for i in self.inputs].index(inplace_of.buf)
        return slot

    # -- variants -------------------------------------------------------------
    def probe(self) -> "Program":
        """Every op output also returned (appended after the normal outputs):
        the unfused schedule used for per-node parity."""
        p = Program()
        p.inputs, p.ops, p.inplace = list(self.inputs), list(self.ops), dict(self.inplace)
        p.outputs = list(self.outputs)
        have = {o.buf for o in self.outputs}
        for op in self.ops:
            if op.out.buf not in have:
                p.outputs.append(op.out)
        p._names = set(self._names)
        return p

    # -- serialisation --------------------------------------------------------
    def text(self) -> str:
        lines = ["tkir 1"]
        for s in self.inputs:
            lines.append(f"in {s.buf} {s.dtype} {_dims_text(s.shape)} {_dims_text(s.strides)} {s.offset}")
        for op in self.ops:
            parts = ["op", op.name, op.opcode, op.out.text()]
            for o in op.operands:
                parts.append(o.text() if isinstance(o, Spec) else hexf(o))
            for k, v in op.attrs.items():
                if k == "dims":
                    parts.append("dims=" + ("all" if v is None else ",".join(str(int(d)) for d in v)))
                else:
                    parts.append(f"{k}={hexf(v)}")
            lines.append(" ".join(parts))
        for s in self.outputs:
            lines.append("out " + s.text())
        for slot, idx in sorted(self.inplace.items()):
            lines.append(f"inplace {slot} {idx}")
        lines.append("end")
        return "\n".join(lines) + "\n"

    def output_shapes(self):
        return [(o.shape, o.dtype) for o in self.outputs]


# ---------------------------------------------------------------------------
# Canonical whole-step programs (forward, MSE loss, explicit backward, SGD).
# ---------------------------------------------------------------------------

def mlp_step(dims, batch: int, dtype: str, lr: float, with_loss: bool = True,
             return_grads: bool = False) -> Program:
    """L-layer MLP, ReLU between layers, MSE loss against t, full backward and an
    in-place SGD update of every weight and bias.  Inputs: x, t, W1, b1, ...

    The backward is written out op by op: gW_i = a_{i-1}^T g_i (transposed view),
    gb_i = sum over the batch, g_{i-1} = threshold_backward(g_i W_i^T, h_{i-1}, 0);
    MSE's gradient is (h_L - t) times fl32(2/(B*d_L)).  Updates use
    ``sub(W, gW, alpha=lr)`` and are returned in place of their inputs.
    """
    L = len(dims) - 1
    p = Program()
    x = p.input("x", dtype, (batch, dims[0]))
    t = p.input("t", dtype, (batch, dims[-1]))
    W, b = [], []
    for i in range(1, L + 1):
        W.append(p.input(f"W{i}", dtype, (dims[i - 1], dims[i])))
        b.append(p.input(f"b{i}", dtype, (dims[i],)))
    a, h = [x], []
    for i in range(L):
        hi = p.op("addmm", [b[i], a[-1], W[i]], dtype, (batch, dims[i + 1]), name=f"h{i + 1}")
        h.append(hi)
        if i < L - 1:
            a.append(p.op("relu", [hi], dtype, name=f"a{i + 1}"))
    d = p.op("sub", [h[-1], t], dtype, name="d")
    loss = None
    if with_loss:
        sq = p.op("pow", [d, 2.0], dtype, name="sq")
        loss = p.op("mean", [sq], dtype, (), name="loss", dims=None)
    g = p.op("mul", [d, f32(2.0 / (batch * dims[-1]))], dtype, name="gy")
    gW, gb = [None] * L, [None] * L
    for i in reversed(range(L)):
        gW[i] = p.op("mm", [a[i].T, g], dtype, (dims[i], dims[i + 1]), name=f"gW{i + 1}")
        gb[i] = p.op("sum", [g], dtype, (dims[i + 1],), name=f"gb{i + 1}", dims=[0])
        if i > 0:
            gm = p.op("mm", [g, W[i].T], dtype, (batch, dims[i]), name=f"gm{i}")
            g = p.op("threshold_backward", [gm, h[i - 1]], dtype, name=f"g{i}", threshold=0.0)
    newW, newb = [], []
    for i in range(L):
        newW.append(p.op("sub", [W[i], gW[i]], dtype, name=f"W{i + 1}_new", alpha=lr))
        newb.append(p.op("sub", [b[i], gb[i]], dtype, name=f"b{i + 1}_new", alpha=lr))
    if loss is not None:
        p.output(loss)
    for i in range(L):
        p.output(newW[i], inplace_of=W[i])
        p.output(newb[i], inplace_of=b[i])
    if return_grads:
        for i in range(L):
            p.output(gW[i])
            p.output(gb[i])
    return p


def residual_step(width: int, layers: int, batch: int, dtype: str, lr: float,
                  with_loss: bool = True, return_grads: bool = False) -> Program:
    """h_i = h_{i-1} + relu(addmm(b_i, h_{i-1}, W_i)), MSE of h_L against t (no
    extra head weight), full backward, in-place SGD.  Inputs: x, t, W1, b1, ..."""
    p = Program()
    x = p.input("x", dtype, (batch, width))
    t = p.input("t", dtype, (batch, width))
    W, b = [], []
    for i in range(1, layers + 1):
        W.append(p.input(f"W{i}", dtype, (width, width)))
        b.append(p.input(f"b{i}", dtype, (width,)))
    hs, zs = [x], []
    for i in range(layers):
        z = p.op("addmm", [b[i], hs[-1], W[i]], dtype, (batch, width), name=f"z{i + 1}")
        zs.append(z)
        r = p.op("relu", [z], dtype, name=f"r{i + 1}")
        hs.append(p.op("add", [hs[-1], r], dtype, name=f"h{i + 1}"))
    d = p.op("sub", [hs[-1], t], dtype, name="d")
    loss = None
    if with_loss:
        sq = p.op("pow", [d, 2.0], dtype, name="sq")
        loss = p.op("mean", [sq], dtype, (), name="loss", dims=None)
    g = p.op("mul", [d, f32(2.0 / (batch * width))], dtype, name="gy")
    gW, gb = [None] * layers, [None] * layers
    for i in reversed(range(layers)):
        gz = p.op("threshold_backward", [g, zs[i]], dtype, name=f"gz{i + 1}", threshold=0.0)
        gW[i] = p.op("mm", [hs[i].T, gz], dtype, (width, width), name=f"gW{i + 1}")
        gb[i] = p.op("sum", [gz], dtype, (width,), name=f"gb{i + 1}", dims=[0])
        if i > 0:
            gm = p.op("mm", [gz, W[i].T], dtype, (batch, width), name=f"gm{i}")
            g = p.op("add", [g, gm], dtype, name=f"g{i}")
    newW, newb = [], []
    for i in range(layers):
        newW.append(p.op("sub", [W[i], gW[i]], dtype, name=f"W{i + 1}_new", alpha=lr))
        newb.append(p.op("sub", [b[i], gb[i]], dtype, name=f"b{i + 1}_new", alpha=lr))
    if loss is not None:
        p.output(loss)
    for i in range(layers):
        p.output(newW[i], inplace_of=W[i])
        p.output(newb[i], inplace_of=b[i])
    if return_grads:
        for i in range(layers):
            p.output(gW[i])
            p.output(gb[i])
    return p


def gemv_q8_stack(k: int, n: int, layers: int, block: int = 32) -> Program:
    """y_l = relu(addmm_q8(b_l, y_{l-1}, q_l, s_l)) in bf16, y_0 = x [1,k].
    q_l is int8 [n,k] (row n holds output n's weights, blocks of ``block``
    along k), s_l float32 [n, ceil(k/block)], b_l float32 [n]."""
    p = Program()
    y = p.input("x", "bf16", (1, k))
    nb = (k + block - 1) // block
    params = []
    for i in range(layers):
        params.append((p.input(f"q{i + 1}", "i8", (n, k)), p.input(f"s{i + 1}", "f32", (n, nb)),
                       p.input(f"b{i + 1}", "f32", (n,))))
    for i, (q, s, b) in enumerate(params):
        z = p.op("addmm_q8", [b, y, q, s], "bf16", (1, n), name=f"z{i + 1}")
        y = p.op("relu", [z], "bf16", name=f"y{i + 1}")
    p.output(y)
    return p


# The five workloads (sizes as stated for the whole-step benchmark set).
CONFIGS = {
    "c1": dict(kind="mlp", dims=(128, 256, 10), batch=64, dtype="f32", lr=0.01),
    "c2": dict(kind="mlp", dims=(512, 1024, 1024, 64), batch=256, dtype="bf16", lr=1e-3),
    "c3": dict(kind="gemv", k=4096, n=4096, layers=8),
    "c4": dict(kind="mlp", dims=(4096, 4096, 4096, 1024), batch=1024, dtype="bf16", lr=1e-4),
    "c5": dict(kind="residual", width=2048, layers=16, batch=512, dtype="f16", lr=1e-4),
}


def build(cfg: dict, **variant) -> Program:
    kind = cfg["kind"]
    if kind == "mlp":
        return mlp_step(cfg["dims"], cfg["batch"], cfg["dtype"], cfg["lr"], **variant)
    if kind == "residual":
        return residual_step(cfg["width"], cfg["layers"], cfg["batch"], cfg["dtype"], cfg["lr"], **variant)
    if kind == "gemv":
        return gemv_q8_stack(cfg["k"], cfg["n"], cfg["layers"])
    raise ValueError(kind)


def inputs_for(cfg: dict, seed: int):
    from . import synth
    kind = cfg["kind"]
    if kind == "mlp":
        return synth.mlp_inputs(seed, cfg["dims"], cfg["batch"], cfg["dtype"])
    if kind == "residual":
        return synth.residual_inputs(seed, cfg["width"], cfg["layers"], cfg["batch"], cfg["dtype"])
    if kind == "gemv":
        return synth.gemv_q8_inputs(seed, cfg["k"], cfg["n"], cfg["layers"])
    raise ValueError(kind)


def contraction_flops(prog: Program) -> int:
    """Sum of 2*m*n*k over the contractions of a program (pointwise work excluded)."""
    total = 0
    for op in prog.ops:
        if op.opcode in ("mm", "mm_q8"):
            a = op.operands[0]
        elif op.opcode in ("addmm", "addmm_q8"):
            a = op.operands[1]
        else:
            continue
        m, k = a.shape
        n = op.out.shape[1]
        total += 2 * m * n * k
    return total


def storage_numpy_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i8": np.int8}[dtype]
