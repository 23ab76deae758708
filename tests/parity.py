"""Parity harness (test infrastructure): run programs through the HIP library
and check them against the CPU oracle.

Tolerance classes (one per op kind):
  * pointwise ops, views, casts, copies, commits: bit-exact (NaN == NaN);
  * contractions (mm, addmm, q8) and reductions (sum, mean, as contractions
    with a ones vector): |gpu - exact| <= 1e-4 * sum_k |a_k||b_k| (plus
    |beta * bias| for addmm, divided by the count for mean), exact = float64;
    a bf16/f16 result also passes within 1 ulp of the oracle's rounded value,
    or within the bound above plus half an ulp of the result (cancellation).

Multi-op programs are checked per node with teacher forcing: the probe variant
returns every op's value; each op is re-evaluated by the oracle from the GPU's
own values of its operands, so accumulation-order differences do not compound.
"""
from __future__ import annotations

import math

import numpy as np

from persistent_whole_step_amd import programs, synth
from persistent_whole_step_amd.programs import Program, Spec, contiguous_strides

TORCH_DT = None


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}[dt]


def to_torch(a: np.ndarray, dt: str, device="cuda:0"):
    from persistent_whole_step_amd import tk
    return tk.tensor_from_storage(a, dt, device)


def to_numpy(t, dt: str) -> np.ndarray:
    from persistent_whole_step_amd import tk
    return tk.storage_from_tensor(t, dt)


def f32_of(a: np.ndarray, dt: str) -> np.ndarray:
    return synth.as_f32(a, dt)


# ------------------------------------------------------------ GPU running --

def gpu_run(prog: Program, inputs, device: int = 0, **opts):
    """Compile for the GPU, run once, return outputs as numpy storage arrays
    (in-place outputs read back from their input tensors)."""
    import torch
    from persistent_whole_step_amd import tk
    p = tk.compile(prog.text(), device=device, **opts)
    ins = [to_torch(a, s.dtype, f"cuda:{device}") for a, s in zip(inputs, prog.inputs)]
    outs = p(*ins)
    torch.cuda.synchronize()
    res = [to_numpy(o, s.dtype) for o, s in zip(outs, prog.outputs)]
    return res, p


# ------------------------------------------------------------- comparison --

def ulp16(v32: np.ndarray, dt: str) -> np.ndarray:
    """Size of one ulp of a bf16/f16 value (normal or subnormal)."""
    mbits = 7 if dt == "bf16" else 10
    emin = -126 if dt == "bf16" else -14
    av = np.abs(v32.astype(np.float64))
    e = np.floor(np.log2(np.where(av > 0, av, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mbits).astype(np.int64))


def assert_bitexact(got: np.ndarray, want: np.ndarray, dt: str, what: str):
    g = f32_of(got, dt)
    w = f32_of(want, dt)
    same = (g.view(np.uint32) == w.view(np.uint32)) | (np.isnan(g) & np.isnan(w))
    if not same.all():
        idx = np.argwhere(~same)[:5]
        raise AssertionError(f"{what}: {int((~same).sum())} of {same.size} differ, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={g[tuple(i)]!r} oracle={w[tuple(i)]!r}" for i in idx))


def assert_contraction(got: np.ndarray, want: np.ndarray, exact: np.ndarray, mag: np.ndarray, dt: str, what: str,
                       rel: float = 1e-4):
    g = f32_of(got, dt).astype(np.float64)
    w = f32_of(want, dt).astype(np.float64)
    bound = rel * mag
    err = np.abs(g - exact)
    ok = err <= bound
    if dt in ("bf16", "f16"):
        u = ulp16(w.astype(np.float32), dt)
        ok |= np.abs(g - w) <= u
        ok |= err <= bound + 0.5 * ulp16(g.astype(np.float32), dt)
    ok |= (np.isnan(g) & np.isnan(exact)) | (np.isinf(g) & (g == exact))
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={g[tuple(i)]!r} exact={exact[tuple(i)]!r} "
                                         f"bound={bound[tuple(i)]!r}" for i in idx))


# -------------------------------------------------- single-op re-evaluation --

def _view_read(buf: np.ndarray, spec: Spec) -> np.ndarray:
    """Values (float64) of a view over a flat buffer (indexing only)."""
    flat = buf.reshape(-1)
    idx = np.full(spec.shape, spec.offset, dtype=np.int64)
    for d, (n, s) in enumerate(zip(spec.shape, spec.strides)):
        shp = [1] * len(spec.shape)
        shp[d] = n
        idx = idx + (np.arange(n, dtype=np.int64) * s).reshape(shp)
    return flat[idx] if flat.size else np.zeros(spec.shape, dtype=flat.dtype)


def single_op_program(prog: Program, j: int, value_specs: dict):
    """A program computing only op j, with each tensor operand's buffer as an input."""
    op = prog.ops[j]
    p = Program()
    names = []
    for a in op.operands:
        if isinstance(a, Spec) and a.buf not in names:
            names.append(a.buf)
    for b in names:
        s = value_specs[b]  # an input spec or an op's (contiguous) output spec
        p.inputs.append(Spec(b, s.dtype, s.shape, s.strides, s.offset))
        p._names.add(b)
    p.ops.append(op)
    p._names.add(op.out.buf)
    p.outputs.append(op.out)
    return p, names


def contraction_reference(op, vals: dict, value_specs: dict):
    """float64 exact value and magnitude sum_k |a||b| (+|beta bias|) of a contraction op."""
    if op.opcode in ("mm", "addmm"):
        A = op.operands[1] if op.opcode == "addmm" else op.operands[0]
        B = op.operands[2] if op.opcode == "addmm" else op.operands[1]
        a = f32_of(_view_read(vals[A.buf], A), A.dtype).astype(np.float64)
        b = f32_of(_view_read(vals[B.buf], B), B.dtype).astype(np.float64)
    else:
        A = op.operands[1] if op.opcode == "addmm_q8" else op.operands[0]
        Q = op.operands[2] if op.opcode == "addmm_q8" else op.operands[1]
        S = op.operands[3] if op.opcode == "addmm_q8" else op.operands[2]
        a = f32_of(_view_read(vals[A.buf], A), A.dtype).astype(np.float64)
        q = _view_read(vals[Q.buf], Q).astype(np.float64)
        s = _view_read(vals[S.buf], S).astype(np.float64)
        k = a.shape[1]
        if op.attrs.get("xq"):
            exact, mag = _xq_reference(a, q, s)
        else:
            w = (q * np.repeat(s, 32, axis=1)[:, :k]).astype(np.float32).astype(np.float64)  # fl(q*s)
            b = w.T
    if op.opcode in ("mm", "addmm") or not op.attrs.get("xq"):
        exact = a @ b
        mag = np.abs(a) @ np.abs(b)
    if op.opcode in ("addmm", "addmm_q8"):
        alpha = op.attrs.get("alpha", 1.0)
        beta = op.attrs.get("beta", 1.0)
        bias = op.operands[0]
        bv = f32_of(_view_read(vals[bias.buf], bias), bias.dtype).astype(np.float64)
        bv = np.broadcast_to(bv, exact.shape)
        exact = alpha * exact + (beta * bv if beta != 0 else 0.0)
        mag = abs(alpha) * mag + (abs(beta) * np.abs(bv) if beta != 0 else 0.0)
    return exact, mag


def xq_codes(a: np.ndarray):
    """Q8_0 codes and block scales of activation rows a [m, k] (float32
    arithmetic: d = amax / 127, codes round-half-even(x / d) in [-127, 127])."""
    a32 = a.astype(np.float32)
    m, k = a32.shape
    nb = (k + 31) // 32
    codes = np.zeros((m, k), np.int64)
    d = np.zeros((m, nb), np.float32)
    for b in range(nb):
        blk = a32[:, 32 * b:32 * b + 32]
        amax = np.abs(blk).max(axis=1)
        db = amax / np.float32(127)
        d[:, b] = db
        nz = db != 0
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.rint(blk / db[:, None])
        codes[nz, 32 * b:32 * b + blk.shape[1]] = np.clip(c[nz], -127, 127).astype(np.int64)
    return codes, d


def _xq_reference(a, q, s):
    """float64 value of the quantised-activation product and its magnitude
    sum_b |d_b s_b| sum_k |code q| (codes from xq_codes)."""
    codes, d = xq_codes(a)
    m, k = a.shape
    n = q.shape[0]
    exact = np.zeros((m, n))
    mag = np.zeros((m, n))
    qi = q.astype(np.int64)
    for b in range(d.shape[1]):
        sl = slice(32 * b, min(k, 32 * b + 32))
        idot = codes[:, sl] @ qi[:, sl].T
        amag = np.abs(codes[:, sl]) @ np.abs(qi[:, sl]).T
        w = (d[:, b][:, None] * s[:, b].astype(np.float32)[None, :]).astype(np.float64)  # fl(d * s)
        exact += w * idot
        mag += np.abs(w) * amag
    return exact, mag


def reduction_reference(op, vals: dict):
    x = op.operands[0]
    xv = f32_of(_view_read(vals[x.buf], x), x.dtype).astype(np.float64)
    dims = op.attrs.get("dims")
    nd = xv.ndim
    axes = tuple(range(nd)) if dims is None else tuple(sorted({d % nd for d in dims})) if nd else ()
    exact = xv.sum(axis=axes) if axes else xv.copy()
    mag = np.abs(xv).sum(axis=axes) if axes else np.abs(xv)
    if op.opcode == "mean":
        cnt = int(np.prod([xv.shape[a] for a in axes])) if axes else 1
        exact = exact / cnt if cnt else exact * np.nan
        mag = mag / max(cnt, 1)
    return np.asarray(exact).reshape(op.out.shape), np.asarray(mag).reshape(op.out.shape)


def check_per_node(oracle_mod, prog: Program, inputs, gpu_vals: dict, ops=None, rel=1e-4):
    """Teacher-forced per-op parity over the probe values `gpu_vals` (buf -> storage array)."""
    value_specs = {s.buf: s for s in prog.inputs}
    for op in prog.ops:
        value_specs[op.out.buf] = op.out
    vals = {s.buf: a for s, a in zip(prog.inputs, inputs)}
    vals.update(gpu_vals)
    checked = 0
    for j, op in enumerate(prog.ops):
        if ops is not None and op.out.buf not in ops:
            continue
        if op.out.buf not in gpu_vals:
            continue
        got = gpu_vals[op.out.buf]
        if op.opcode in programs.POINTWISE:
            sp, names = single_op_program(prog, j, value_specs)
            (want,) = oracle_mod.run(sp.text(), [np.ascontiguousarray(vals[n]) for n in names])
            assert_bitexact(got, want, op.out.dtype, f"{op.name} ({op.opcode})")
        else:
            sp, names = single_op_program(prog, j, value_specs)
            (want,) = oracle_mod.run(sp.text(), [np.ascontiguousarray(vals[n]) for n in names])
            if op.opcode in programs.REDUCTIONS:
                exact, mag = reduction_reference(op, vals)
            else:
                exact, mag = contraction_reference(op, vals, value_specs)
            assert_contraction(got.reshape(op.out.shape), want.reshape(op.out.shape), exact, mag, op.out.dtype,
                               f"{op.name} ({op.opcode})", rel)
        checked += 1
    return checked


def probe_values(prog: Program, probe: Program, outs):
    """Map buffer name -> GPU value from a probe run's outputs (skip in-place slots
    whose values are the updated inputs: those are named by their op buffer too)."""
    vals = {}
    for spec, v in zip(probe.outputs, outs):
        vals[spec.buf] = v
    return vals


# ------------------------------------------- full sizes: sampled contractions --

def _gather(buf: np.ndarray, spec: Spec, idx) -> np.ndarray:
    """Elements of view `spec` at index arrays idx[d] (one per view dim), from
    the flat buffer `buf` (indexing only)."""
    flat = buf.reshape(-1)
    pos = np.full(np.broadcast(*idx).shape if idx else (), spec.offset, dtype=np.int64)
    for d, c in enumerate(idx):
        pos = pos + np.asarray(c, dtype=np.int64) * spec.strides[d]
    return flat[pos]


def tile_cover(n: int, rng, block: int = 64) -> np.ndarray:
    """Sorted, unique indices into a dimension of size n: one random index
    inside every block of `block` consecutive indices (the last block may be
    short), plus the first and the last index.  Sampling rows and columns this
    way puts at least one sampled output in every output tile of any tiling
    whose tile edges are multiples of `block` (64x64 and 128x128 tiles)."""
    if n <= 0:
        return np.zeros(0, np.int64)
    starts = np.arange(0, n, block)
    ends = np.minimum(starts + block, n)
    picks = starts + (rng.random(len(starts)) * (ends - starts)).astype(np.int64)
    return np.unique(np.concatenate([[0, n - 1], picks]).astype(np.int64))


def _bias_block(buf: np.ndarray, spec: Spec, rows, cols) -> np.ndarray:
    """A bias view broadcast over an [m, n] output, read at every (rows[i],
    cols[j]) (indexing only): an array [len(rows), len(cols)]."""
    r = len(spec.shape)
    full = (np.asarray(rows)[:, None], np.asarray(cols)[None, :])
    idx = []
    for d in range(r):
        c = full[2 - r + d]
        idx.append(np.zeros_like(c) if spec.shape[d] == 1 else c)
    shape = (len(rows), len(cols))
    return np.broadcast_to(_gather(buf, spec, idx), shape).copy()


def sampled_contraction_program(op, vals: dict, rows, cols):
    """A small program whose output (i, j) is op's output at (rows[i],
    cols[j]): the sampled rows of the activation operand, the sampled columns
    (output features) of the weight operand, and the bias read at every
    sampled output.  Each output of a contraction depends on its own row and
    column only, so the oracle's value there is the value it computes for the
    full op."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    sr, sc = len(rows), len(cols)
    p = Program()
    arrays = []
    bias_first = op.opcode in ("addmm", "addmm_q8")
    ops_in = op.operands[1:] if bias_first else op.operands
    if op.opcode in ("mm", "addmm"):
        A, B = ops_in
        k = A.shape[1]
        kk = np.arange(k)
        a = _gather(vals[A.buf], A, (rows[:, None], kk[None, :]))
        b = _gather(vals[B.buf], B, (kk[:, None], cols[None, :]))
        sa = p.input("A", A.dtype, (sr, k))
        sb = p.input("B", B.dtype, (k, sc))
        operands = [sa, sb]
        arrays += [np.ascontiguousarray(a), np.ascontiguousarray(b)]
    else:
        X, Q, S = ops_in
        k = X.shape[1]
        kk = np.arange(k)
        nb = S.shape[1]
        x = _gather(vals[X.buf], X, (rows[:, None], kk[None, :]))
        q = _gather(vals[Q.buf], Q, (cols[:, None], kk[None, :]))
        sc_ = _gather(vals[S.buf], S, (cols[:, None], np.arange(nb)[None, :]))
        sx = p.input("x", X.dtype, (sr, k))
        sq = p.input("q", Q.dtype, (sc, k))
        ss = p.input("s", S.dtype, (sc, nb))
        operands = [sx, sq, ss]
        arrays += [np.ascontiguousarray(x), np.ascontiguousarray(q), np.ascontiguousarray(sc_)]
    if bias_first:
        Bi = op.operands[0]
        sbias = p.input("bias", Bi.dtype, (sr, sc))
        operands = [sbias] + operands
        arrays = arrays + [np.ascontiguousarray(_bias_block(vals[Bi.buf], Bi, rows, cols))]
    out = p.op(op.opcode, operands, op.out.dtype, (sr, sc), name="y", **op.attrs)
    p.output(out)
    return p, arrays


def check_per_node_sampled(oracle_mod, prog: Program, inputs, gpu_vals: dict, seed: int = 0, rel=1e-4,
                           block: int = 64):
    """Teacher-forced per-op parity at full size: pointwise ops and reductions
    are re-evaluated whole by the oracle (bit-exact / contraction tolerance);
    each contraction is checked on the block of outputs at the rows and
    columns `tile_cover` picks (one in every 64 along each dimension, and the
    edges), so every output tile holds checked outputs.  Each checked output
    is computed by the oracle from the GPU's own operand values and compared
    with its exact float64 value."""
    rng = np.random.default_rng(seed)
    value_specs = {s.buf: s for s in prog.inputs}
    for op in prog.ops:
        value_specs[op.out.buf] = op.out
    vals = {s.buf: a for s, a in zip(prog.inputs, inputs)}
    vals.update(gpu_vals)
    checked = 0
    for j, op in enumerate(prog.ops):
        if op.out.buf not in gpu_vals:
            continue
        got = gpu_vals[op.out.buf]
        if op.opcode in programs.CONTRACTIONS:
            m, n = op.out.shape
            rows, cols = tile_cover(m, rng, block), tile_cover(n, rng, block)
            sp, arrays = sampled_contraction_program(op, vals, rows, cols)
            (want,) = oracle_mod.run(sp.text(), arrays)
            svals = {s.buf: a for s, a in zip(sp.inputs, arrays)}
            exact, mag = contraction_reference(sp.ops[0], svals, None)
            g = got.reshape(m, n)[rows[:, None], cols[None, :]]
            assert_contraction(g, want.reshape(len(rows), len(cols)), exact, mag, op.out.dtype,
                               f"{op.name} ({op.opcode}, {len(rows)}x{len(cols)} sampled outputs)", rel)
        else:
            sp, names = single_op_program(prog, j, value_specs)
            (want,) = oracle_mod.run(sp.text(), [np.ascontiguousarray(vals[nm]) for nm in names])
            if op.opcode in programs.POINTWISE:
                assert_bitexact(got, want, op.out.dtype, f"{op.name} ({op.opcode})")
            else:
                exact, mag = reduction_reference(op, vals)
                assert_contraction(got.reshape(op.out.shape), want.reshape(op.out.shape), exact, mag, op.out.dtype,
                                   f"{op.name} ({op.opcode})", rel)
        checked += 1
    return checked
