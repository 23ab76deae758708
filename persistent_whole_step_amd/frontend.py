"""Capture a PyTorch training step into a whole-step program.

The runtime page's README describes the front end this mirrors:
``capture(fn, examples)`` returns the program of a step function (usable
without a GPU, for inspection), and ``compile_training(fn, examples)`` compiles
a step written with ``torch.func.grad_and_value`` into one persistent launch,
checking that the gradients mirror the state tree and deriving which outputs
update the state in place.  The page does not show the front end's source;
this one is written from that description.

Tracing uses PyTorch's own tracer (``make_fx``), which turns the step,
gradient transforms included, into ATen operations.  Each ATen operation maps
onto the program's op set (mm, addmm, the pointwise ops, sum/mean, views);
anything else is rejected with the operation's name.  The captured program is
then an ordinary input of the C-ABI library: every arithmetic step runs in
the HIP kernel.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import programs
from .programs import Program, Spec, contiguous_strides


def _dtype_name(dt) -> str:
    import torch
    names = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.int8: "i8"}
    if dt not in names:
        raise TypeError(f"capture: unsupported dtype {dt}")
    return names[dt]


def _scalar(v) -> float:
    if isinstance(v, bool) or not isinstance(v, (int, float)):
        raise TypeError(f"capture: expected a number, got {v!r}")
    return float(v)


def _is_contiguous(s: Spec) -> bool:
    return s.offset >= 0 and tuple(s.strides) == contiguous_strides(s.shape)


class _Lowering:
    """ATen graph -> Program, one node at a time."""

    def __init__(self, prog: Program):
        self.p = prog
        self.env = {}

    def val(self, a):
        """A node argument: a Spec (tensor value) or a Python number."""
        import torch.fx
        if isinstance(a, torch.fx.Node):
            return self.env[a]
        return _scalar(a)

    def emit(self, node, opcode, operands, **attrs):
        meta = node.meta["val"]
        return self.p.op(opcode, operands, _dtype_name(meta.dtype), tuple(meta.shape), name=node.name, **attrs)

    def lower(self, node):
        import torch
        aten = torch.ops.aten
        t = node.target
        a = node.args
        meta = node.meta.get("val")
        shape = tuple(meta.shape) if meta is not None else None
        # views: no op, a new view of the same buffer
        if t in (aten.t.default, aten.transpose.int, aten.permute.default):
            x = self.val(a[0])
            r = len(x.shape)
            if t == aten.permute.default:
                perm = [int(d) % max(r, 1) for d in a[1]]
                if sorted(perm) != list(range(r)):
                    raise NotImplementedError(f"capture: permute dims {list(a[1])} of a rank-{r} tensor")
            else:
                if t == aten.t.default:
                    if r > 2:
                        raise NotImplementedError(f"capture: t() of a rank-{r} tensor")
                    d0, d1 = (0, 1) if r == 2 else (0, 0)
                else:
                    d0, d1 = int(a[1]) % max(r, 1), int(a[2]) % max(r, 1)
                perm = list(range(r))
                if r:
                    perm[d0], perm[d1] = perm[d1], perm[d0]
            if perm == list(range(r)):  # the identity permutation: the same view
                return x
            return x.view(tuple(x.shape[d] for d in perm), tuple(x.strides[d] for d in perm), x.offset)
        if t in (aten.view.default, aten._unsafe_view.default, aten.reshape.default):
            x = self.val(a[0])
            if not _is_contiguous(x):
                raise NotImplementedError(f"capture: {t} of a non-contiguous view")
            return x.view(shape, contiguous_strides(shape), x.offset)
        if t in (aten.unsqueeze.default, aten.squeeze.dim):
            x = self.val(a[0])
            r = len(x.shape)
            if t == aten.unsqueeze.default:
                d = int(a[1]) % (r + 1)
                return x.view(x.shape[:d] + (1,) + x.shape[d:], x.strides[:d] + (0,) + x.strides[d:], x.offset)
            d = int(a[1]) % max(r, 1)
            if r == 0 or x.shape[d] != 1:
                return x
            return x.view(x.shape[:d] + x.shape[d + 1:], x.strides[:d] + x.strides[d + 1:], x.offset)
        if t == aten.expand.default:
            x = self.val(a[0])
            r = len(shape) - len(x.shape)
            strides = [0] * r
            for d, n in enumerate(x.shape):
                strides.append(0 if n == 1 and shape[r + d] != 1 else x.strides[d])
            return x.view(shape, strides, x.offset)
        if t in (aten.detach.default, aten.alias.default, aten.lift_fresh_copy.default):
            return self.val(a[0])
        # element-wise
        if t in (aten.add.Tensor, aten.sub.Tensor):
            x, y = self.val(a[0]), self.val(a[1])
            alpha = _scalar(node.kwargs.get("alpha", 1))
            op = "add" if t == aten.add.Tensor else "sub"
            if not isinstance(x, Spec):  # a scalar first operand becomes a filled tensor
                x = self._full(node, x)
            attrs = {"alpha": alpha} if alpha != 1.0 else {}
            return self.emit(node, op, [x, y], **attrs)
        if t in (aten.mul.Tensor, aten.mul.Scalar):
            x, y = self.val(a[0]), self.val(a[1])
            if not isinstance(x, Spec):
                x, y = y, x
            return self.emit(node, "mul", [x, y])
        if t in (aten.div.Tensor, aten.div.Scalar):
            x, y = self.val(a[0]), self.val(a[1])
            if not isinstance(x, Spec):
                x = self._full(node, x)
            return self.emit(node, "div", [x, y])
        if t == aten.neg.default:
            return self.emit(node, "neg", [self.val(a[0])])
        if t == aten.relu.default:
            return self.emit(node, "relu", [self.val(a[0])])
        if t == aten.sqrt.default:
            return self.emit(node, "sqrt", [self.val(a[0])])
        if t == aten.pow.Tensor_Scalar:
            x, e = self.val(a[0]), _scalar(a[1])
            if e == 1.0:  # x ** 1 is x exactly: a rounding to the result dtype only
                return self.emit(node, "cast", [x])
            return self.emit(node, "pow", [x, e])
        if t == aten.threshold_backward.default:
            g, x, thr = self.val(a[0]), self.val(a[1]), _scalar(a[2])
            return self.emit(node, "threshold_backward", [g, x], threshold=thr)
        if t in (aten._to_copy.default, aten.clone.default):
            return self.emit(node, "cast", [self.val(a[0])])
        if t in (aten.ones_like.default, aten.zeros_like.default, aten.full_like.default):
            value = 1.0 if t == aten.ones_like.default else 0.0 if t == aten.zeros_like.default else _scalar(a[1])
            return self.emit(node, "full", [], value=value)
        if t in (aten.full.default, aten.scalar_tensor.default):
            value = _scalar(a[1] if t == aten.full.default else a[0])
            return self.emit(node, "full", [], value=value)
        # contractions
        if t == aten.mm.default:
            return self.emit(node, "mm", [self.val(a[0]), self.val(a[1])])
        if t == aten.addmm.default:
            bias, x, w = self.val(a[0]), self.val(a[1]), self.val(a[2])
            beta = _scalar(node.kwargs.get("beta", 1))
            alpha = _scalar(node.kwargs.get("alpha", 1))
            return self.emit(node, "addmm", [bias, x, w], alpha=alpha, beta=beta)
        # reductions
        if t in (aten.sum.dim_IntList, aten.mean.dim, aten.sum.default, aten.mean.default):
            x = self.val(a[0])
            op = "sum" if t in (aten.sum.dim_IntList, aten.sum.default) else "mean"
            if t in (aten.sum.default, aten.mean.default):
                dims, keep = None, False
            else:
                dims = [int(d) for d in a[1]] if a[1] is not None else None
                keep = bool(a[2]) if len(a) > 2 else bool(node.kwargs.get("keepdim", False))
            rank = len(x.shape)
            red = set(range(rank)) if dims is None else {d % rank for d in dims}
            out_shape = tuple(n for d, n in enumerate(x.shape) if d not in red)
            out = self.p.op(op, [x], _dtype_name(meta.dtype), out_shape, name=node.name,
                            dims=None if dims is None else sorted(red))
            if keep:
                return out.view(shape, contiguous_strides(shape), 0)
            return out
        raise NotImplementedError(f"capture: no program op for {t}")

    def _full(self, node, v):
        meta = node.meta["val"]
        return self.p.op("full", [], _dtype_name(meta.dtype), tuple(meta.shape), name=node.name + "_scalar",
                         value=float(v))


@dataclass
class Captured:
    """A captured step: the program, the input and output tree specs, and the
    output leaves' positions."""
    program: Program
    in_spec: object
    out_spec: object


def capture(fn, examples):
    """Trace ``fn(*examples)`` (tensors in nested tuples, lists and dicts) and
    return (program, output tree spec).  Needs no GPU: the examples may be CPU
    tensors.  Every example tensor must be contiguous; the program's inputs
    are the flattened example leaves in order."""
    c = _capture(fn, examples)
    return c.program, c.out_spec


def _capture(fn, examples) -> Captured:
    import torch
    from torch.fx.experimental.proxy_tensor import make_fx
    from torch.utils import _pytree as pytree
    leaves, in_spec = pytree.tree_flatten(tuple(examples))
    for i, leaf in enumerate(leaves):
        if not isinstance(leaf, torch.Tensor):
            raise TypeError(f"capture: example leaf {i} is not a tensor")
        if not leaf.is_contiguous():
            raise ValueError(f"capture: example leaf {i} must be contiguous")
    out_spec_box = []

    def flat_fn(*xs):
        outs = fn(*pytree.tree_unflatten(list(xs), in_spec))
        flat, spec = pytree.tree_flatten(outs)
        out_spec_box.append(spec)
        return flat

    gm = make_fx(flat_fn, tracing_mode="fake")(*leaves)
    p = Program()
    low = _Lowering(p)
    ph = 0
    out_nodes = None
    for node in gm.graph.nodes:
        if node.op == "placeholder":
            leaf = leaves[ph]
            low.env[node] = p.input(f"in{ph}", _dtype_name(leaf.dtype), tuple(leaf.shape))
            ph += 1
        elif node.op == "call_function":
            low.env[node] = low.lower(node)
        elif node.op == "output":
            out_nodes = node.args[0]
        else:
            raise NotImplementedError(f"capture: graph node kind {node.op}")
    for o in out_nodes:
        v = low.env[o]
        if not isinstance(v, Spec):
            raise NotImplementedError("capture: outputs must be tensors")
        p.output(v)
    return Captured(p, in_spec, out_spec_box[-1])


def _update_mapping(c: Captured):
    """In-place pairs {output slot: input index} for the updated state.  The
    state is the first argument's tree; the updated state is the last output
    subtree with the same structure whose every leaf is an update of the
    matching state leaf: an add or sub (w - lr * g, or an optimizer state's
    beta * m + (1 - beta) * g) whose chain of first operands, through
    pointwise ops, leads back to that leaf, with its shape and dtype.  The
    gradients (the same structure, produced otherwise) stay ordinary
    outputs."""
    from torch.utils import _pytree as pytree
    p = c.program
    first = pytree.tree_unflatten(list(range(len(p.inputs))), c.in_spec)[0]
    state_leaves, state_spec = pytree.tree_flatten(first)
    out_idx = pytree.tree_unflatten(list(range(len(p.outputs))), c.out_spec)
    producers = {op.out.buf: op for op in p.ops}

    def updates(buf: str, src: str) -> bool:
        op = producers.get(buf)
        if op is None or op.opcode not in ("add", "sub"):
            return False
        seen = 0
        while op is not None and seen < 64:
            head = op.operands[0] if op.operands else None
            if not isinstance(head, Spec):
                return False
            if head.buf == src:
                return True
            op = producers.get(head.buf)
            if op is not None and op.opcode not in programs.POINTWISE:
                return False
            seen += 1
        return False

    def candidates(tree):
        leaves, spec = pytree.tree_flatten(tree)
        if spec == state_spec:
            yield leaves
        if isinstance(tree, (tuple, list)):
            for sub in tree:
                yield from candidates(sub)
        elif isinstance(tree, dict):
            for sub in tree.values():
                yield from candidates(sub)

    best = None
    for leaves in candidates(out_idx):
        ok = True
        for slot, si in zip(leaves, state_leaves):
            o, src = p.outputs[slot], p.inputs[si]
            if o.shape != src.shape or o.dtype != src.dtype or not updates(o.buf, src.buf):
                ok = False
                break
        if ok:
            best = leaves
    if best is None or len(set(best)) != len(best) or len(best) != len(state_leaves):
        return {}
    return {slot: si for slot, si in zip(best, state_leaves)}


class CompiledTrainingStep:
    """One compiled step: call it with arguments of the example's tree, shapes,
    strides and dtypes; returns the step's output tree.  Updated state is
    written into the state tensors passed in (they must not require grad) and
    those same tensors are returned in its place."""

    def __init__(self, captured: Captured, inplace: dict, device: int, **opts):
        from . import tk
        self.captured = captured
        self.program = captured.program
        self.program.inplace = dict(inplace)
        self.compiled = tk.compile(self.program.text(), device=device, **opts)

    def __call__(self, *args):
        from torch.utils import _pytree as pytree
        leaves, spec = pytree.tree_flatten(tuple(args))
        if spec != self.captured.in_spec:
            raise TypeError("compiled step: arguments do not match the captured tree")
        outs = self.compiled(*leaves)
        return pytree.tree_unflatten(list(outs), self.captured.out_spec)

    def query(self) -> dict:
        return self.compiled.query()

    def capture(self, *args, warmup: int = 2) -> "CapturedProgram":
        """A reusable graph of one step on these arguments (the runtime page
        README's ``compiled.capture``): ``warmup`` eager steps, then one
        launch captured into a HIP graph; the state tensors are restored to
        the values they held on entry after warmup and capture.  Replays run
        the step on the same tensors: the state advances in place, and other
        outputs live in buffers allocated here (fixed shapes and addresses,
        overwritten by every replay)."""
        import torch
        from torch.utils import _pytree as pytree
        from . import tk
        leaves, spec = pytree.tree_flatten(tuple(args))
        if spec != self.captured.in_spec:
            raise TypeError("compiled step: arguments do not match the captured tree")
        prog = self.compiled
        if getattr(prog, "launch_mode", 0) != 1:
            # graph capture records ordinary launches only
            prog = tk.compile(self.program.text(), device=self.compiled.device, launch_mode=1)
        targets = sorted(set(self.program.inplace.values()))
        saved = {i: leaves[i].detach().clone() for i in targets}
        bufs = prog.allocate(*leaves)
        for _ in range(max(0, int(warmup))):
            prog.run_into(*leaves, buffers=bufs)
        torch.cuda.synchronize()
        graph = tk.StepGraph(prog, [(leaves, bufs)])
        for i, v in saved.items():
            leaves[i].copy_(v)
        torch.cuda.synchronize()
        return CapturedProgram(graph, bufs, self.captured.out_spec)


class CapturedProgram:
    """A captured step (see ``CompiledTrainingStep.capture``).  ``replay()``
    enqueues one step on the current stream and returns the output tree,
    whose tensors are the captured buffers and state tensors."""

    def __init__(self, graph, buffers, out_spec):
        self.graph = graph
        self.buffers = buffers
        self.out_spec = out_spec

    def replay(self):
        from torch.utils import _pytree as pytree
        self.graph.replay()
        return pytree.tree_unflatten(list(self.buffers.outputs), self.out_spec)


def compile_training(fn, examples, device: int = 0, inplace: bool = True, **opts) -> CompiledTrainingStep:
    """Capture ``fn`` on ``examples`` and compile it for the GPU.  With
    ``inplace``, the updated state (see ``_update_mapping``) is committed into
    the state tensors; it needs the state's gradients to mirror its tree."""
    c = _capture(fn, examples)
    mapping = _update_mapping(c) if inplace else {}
    return CompiledTrainingStep(c, mapping, device, **opts)
