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

POINTWISE = ("add", "sub", "mul", "div", "neg", "relu", "pow", "threshold_backward", "full", "cast", "sqrt")
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
# Parameter updates.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AdamW:
    """Adam with decoupled weight decay (Loshchilov and Hutter), the optimizer
    the trainkernel README's roadmap names next after SGD.

    Hyper-parameters are static scalars of the program.  The step-dependent
    bias corrections are not: they enter as two one-element float32 inputs,
    ``c1 = 1/(1 - beta1^t)`` and ``c2 = 1/(1 - beta2^t)``, so one compiled
    program serves every step t (the caller recomputes them per step)."""
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 1e-2

    def corrections(self, t: int):
        """(c1, c2) for step t >= 1, each rounded once to float32."""
        if t < 1:
            raise ValueError("AdamW steps count from 1")
        return f32(1.0 / (1.0 - self.beta1 ** t)), f32(1.0 / (1.0 - self.beta2 ** t))


def adamw_update(p: Program, w: Spec, g: Spec, m: Spec, v: Spec, c1: Spec, c2: Spec,
                 lr: float, opt: AdamW, name: str):
    """One parameter's AdamW update, written as pointwise ops evaluated in
    float32 (states m and v are float32; the gradient is widened on read):

        w_d = w * (1 - lr*wd)                 decoupled decay, applied first
        m'  = beta1*m + (1-beta1)*g
        v'  = beta2*v + (1-beta2)*(g*g)
        w'  = w_d - lr * (m'*c1) / (sqrt(v'*c2) + eps)    rounded to w's dtype

    Returns (w', m', v')."""
    sh = w.shape
    one = lambda s: s.view(sh, (0,) * len(sh))  # broadcast a one-element input
    wd = p.op("mul", [w, f32(1.0 - lr * opt.weight_decay)], "f32", sh, name=f"{name}_decayed")
    m1 = p.op("mul", [m, f32(opt.beta1)], "f32", sh, name=f"{name}_m_decay")
    mn = p.op("add", [m1, g], "f32", sh, name=f"{name}_m_new", alpha=f32(1.0 - opt.beta1))
    gg = p.op("mul", [g, g], "f32", sh, name=f"{name}_g_sq")
    v1 = p.op("mul", [v, f32(opt.beta2)], "f32", sh, name=f"{name}_v_decay")
    vn = p.op("add", [v1, gg], "f32", sh, name=f"{name}_v_new", alpha=f32(1.0 - opt.beta2))
    mh = p.op("mul", [mn, one(c1)], "f32", sh, name=f"{name}_m_hat")
    vh = p.op("mul", [vn, one(c2)], "f32", sh, name=f"{name}_v_hat")
    rt = p.op("sqrt", [vh], "f32", sh, name=f"{name}_v_root")
    dn = p.op("add", [rt, f32(opt.eps)], "f32", sh, name=f"{name}_denom")
    u = p.op("div", [mh, dn], "f32", sh, name=f"{name}_step")
    wn = p.op("sub", [wd, u], w.dtype, sh, name=f"{name}_new", alpha=f32(lr))
    return wn, mn, vn


def _update(p: Program, weights, biases, loss, dtype: str, lr: float, optimizer, return_grads: bool):
    """Append the parameter update and the outputs: loss, then (W_i', b_i') per
    layer in place of W_i, b_i, then with AdamW (m', v') of W1, b1, W2, ... in
    place of their states, then the gradients when asked for.  AdamW adds the
    inputs m and v (float32, parameter-shaped) per parameter in the same order,
    then c1 and c2."""
    pairs = [x for wb in zip(weights, biases) for x in wb]
    new, states = [], []
    if optimizer is None:
        for w, g, nm in pairs:
            new.append(p.op("sub", [w, g], dtype, name=f"{nm}_new", alpha=lr))
    else:
        mv = [(p.input(f"m_{nm}", "f32", w.shape), p.input(f"v_{nm}", "f32", w.shape)) for w, _, nm in pairs]
        c1 = p.input("c1", "f32", (1,))
        c2 = p.input("c2", "f32", (1,))
        for (w, g, nm), (m, v) in zip(pairs, mv):
            wn, mn, vn = adamw_update(p, w, g, m, v, c1, c2, lr, optimizer, nm)
            new.append(wn)
            states.append((mn, m, vn, v))
    if loss is not None:
        p.output(loss)
    for (w, _, _), wn in zip(pairs, new):
        p.output(wn, inplace_of=w)
    for mn, m, vn, v in states:
        p.output(mn, inplace_of=m)
        p.output(vn, inplace_of=v)
    if return_grads:
        for _, g, _ in pairs:
            p.output(g)


# ---------------------------------------------------------------------------
# Canonical whole-step programs (forward, MSE loss, explicit backward, SGD).
# ---------------------------------------------------------------------------

def mlp_step(dims, batch: int, dtype: str, lr: float, with_loss: bool = True,
             return_grads: bool = False, optimizer: "AdamW | None" = None) -> Program:
    """L-layer MLP, ReLU between layers, MSE loss against t, full backward and an
    in-place SGD update of every weight and bias.  Inputs: x, t, W1, b1, ...

    The backward is written out op by op: gW_i = a_{i-1}^T g_i (transposed view),
    gb_i = sum over the batch, g_{i-1} = threshold_backward(g_i W_i^T, h_{i-1}, 0);
    MSE's gradient is (h_L - t) times fl32(2/(B*d_L)).  Updates use
    ``sub(W, gW, alpha=lr)`` and are returned in place of their inputs; with an
    ``AdamW`` optimizer the update is the one ``adamw_update`` writes out.
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
    _update(p, [(W[i], gW[i], f"W{i + 1}") for i in range(L)], [(b[i], gb[i], f"b{i + 1}") for i in range(L)],
            loss, dtype, lr, optimizer, return_grads)
    return p


def residual_step(width: int, layers: int, batch: int, dtype: str, lr: float,
                  with_loss: bool = True, return_grads: bool = False,
                  optimizer: "AdamW | None" = None) -> Program:
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
    _update(p, [(W[i], gW[i], f"W{i + 1}") for i in range(layers)],
            [(b[i], gb[i], f"b{i + 1}") for i in range(layers)], loss, dtype, lr, optimizer, return_grads)
    return p


def gemv_q8_stack(k: int, n: int, layers: int, block: int = 32, rows: int = 1, xq: bool = False) -> Program:
    """y_l = relu(addmm_q8(b_l, y_{l-1}, q_l, s_l)) in bf16, y_0 = x [rows,k]
    (rows > 1: several decode rows sharing each weight pass).
    q_l is int8 [n,k] (row n holds output n's weights, blocks of ``block``
    along k), s_l float32 [n, ceil(k/block)], b_l float32 [n].
    xq: each product first quantises its activation rows to Q8_0 (blocks of
    32, one float32 scale each) and multiplies codes by codes."""
    p = Program()
    y = p.input("x", "bf16", (rows, k))
    nb = (k + block - 1) // block
    params = []
    for i in range(layers):
        params.append((p.input(f"q{i + 1}", "i8", (n, k)), p.input(f"s{i + 1}", "f32", (n, nb)),
                       p.input(f"b{i + 1}", "f32", (n,))))
    for i, (q, s, b) in enumerate(params):
        z = p.op("addmm_q8", [b, y, q, s], "bf16", (rows, n), name=f"z{i + 1}", **({"xq": 1.0} if xq else {}))
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
    opt = cfg.get("optimizer")
    if opt is not None:
        variant.setdefault("optimizer", opt)
    if kind == "mlp":
        return mlp_step(cfg["dims"], cfg["batch"], cfg["dtype"], cfg["lr"], **variant)
    if kind == "residual":
        return residual_step(cfg["width"], cfg["layers"], cfg["batch"], cfg["dtype"], cfg["lr"], **variant)
    if kind == "gemv":
        return gemv_q8_stack(cfg["k"], cfg["n"], cfg["layers"], rows=cfg.get("rows", 1), xq=cfg.get("xq", False))
    raise ValueError(kind)


def inputs_for(cfg: dict, seed: int):
    from . import synth
    kind = cfg["kind"]
    opt = cfg.get("optimizer")
    if kind == "mlp":
        base = synth.mlp_inputs(seed, cfg["dims"], cfg["batch"], cfg["dtype"])
    elif kind == "residual":
        base = synth.residual_inputs(seed, cfg["width"], cfg["layers"], cfg["batch"], cfg["dtype"])
    else:
        base = None
    if base is not None:
        if opt is None:
            return base
        c1, c2 = opt.corrections(cfg.get("adam_t", 10))
        return (base + synth.adamw_state(seed + 1, [a.shape for a in base[2:]])
                + [np.array([c1], np.float32), np.array([c2], np.float32)])
    if kind == "gemv":
        return synth.gemv_q8_inputs(seed, cfg["k"], cfg["n"], cfg["layers"], rows=cfg.get("rows", 1))
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
