"""Schedule race checker for compiled plans (host only, no GPU).

Reads the device plan that tk_compile uploads (tk_plan_bytes; the structs of
csrc/plan.h) and, for every stage, derives each work item's reads and writes
from the descriptors the kernel interprets: contraction tiles (operand rows
and columns over their K range, epilogue views over the tile), one-row
products (slab rows and columns), elementwise items (4096 elements of the
iteration space), row and column reductions (their rows, parts and partial
slots), split-K and reduction combines.  Items of one stage run concurrently
on different workgroups, so a write of one item that touches bytes another
item of the same stage reads or writes is a race; the grid barrier between
two stages is what orders them.

The codegen page's generator guards its schedule with a static hazard pass
over read and write regions (trainkernel codegen.py, `_Generator.generate`);
this checker re-derives the regions from the encoded plan instead of from the
scheduler's own bookkeeping, so it also catches a descriptor that does not
mean what the scheduler intended.  `merge` joins stages (drops barriers):
dropping a barrier the schedule needs must produce a race.

Regions are compared first as byte intervals (bounding boxes per item and
view), and every overlapping pair is then confirmed on the exact element
addresses, so strided and transposed views do not produce false reports.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass, field

import numpy as np

# csrc/plan.h
T_EW, T_GEMM_MFMA, T_GEMM_SIMT, T_GEMM_REDUCE, T_GEMV_Q8, T_GEMV, T_RED_ROWS, T_RED_COLS, T_RED_FINAL = range(1, 10)
F_PARTIAL, F_ROWWG, F_COLLANES32, F_BSUM = 2, 4, 256, 512  # plan.h flags
VM_STORE = 12
SRC_VIEW = 1
KBLOCK = 256
GEMV_ROWS = 4
ESIZE = {0: 4, 1: 2, 2: 2, 3: 1}

_TASK = struct.Struct("<BBBBI6I4I4I4B3I4I4HQfI2I")
_VIEW = struct.Struct("<q4qHB5x")
_INS = struct.Struct("<BBBBHHff")
_STAGE = struct.Struct("<8I")
_HEADER = struct.Struct("<8I")


@dataclass
class Task:
    kind: int
    width: int
    ndim: int
    tile: int
    flags: int
    n_items: int
    item_begin: int
    expr_first: int
    expr_len: int
    fin_first: int
    fin_len: int
    dims: tuple
    m: int
    n: int
    k: int
    split: int
    kchunk: int
    tiles_m: int
    tiles_n: int
    va: int
    vb: int
    vs: int
    vx: int
    scratch: int
    bs_first: int = 0
    bs_len: int = 0


@dataclass
class View:
    offset: int
    strides: tuple
    base: int
    dtype: int


@dataclass
class Stage:
    tasks: list
    views: list
    ins: list  # (op, src, arg)
    n_items: int


def decode(plan: bytes) -> list:
    """The stages of an encoded plan."""
    magic, n_stages, off_stages, nbytes = _HEADER.unpack_from(plan, 0)[:4]
    if magic != 0x31706B74:
        raise ValueError("not a tk plan")
    assert _TASK.size == 128 and _VIEW.size == 48 and _INS.size == 16
    stages = []
    for s in range(n_stages):
        blob_off, blob_bytes, n_tasks, n_items, off_views, off_ins, n_views, n_ins = _STAGE.unpack_from(
            plan, off_stages + 32 * s)
        tasks = []
        for i in range(n_tasks):
            f = _TASK.unpack_from(plan, blob_off + i * _TASK.size)
            tasks.append(Task(kind=f[0], width=f[1], ndim=f[2], tile=f[3], flags=f[4], n_items=f[5],
                              item_begin=f[6], expr_first=f[7], expr_len=f[8], fin_first=f[9], fin_len=f[10],
                              dims=tuple(f[11:15]), m=f[23], n=f[24], k=f[25], split=f[26], kchunk=f[27],
                              tiles_m=f[28], tiles_n=f[29], va=f[30], vb=f[31], vs=f[32], vx=f[33],
                              scratch=f[34], bs_first=f[37], bs_len=f[38]))
        assert off_views >= n_tasks * _TASK.size
        views = []
        for i in range(n_views):
            f = _VIEW.unpack_from(plan, blob_off + off_views + i * _VIEW.size)
            views.append(View(offset=f[0], strides=tuple(f[1:5]), base=f[5], dtype=f[6]))
        ins = []
        for i in range(n_ins):
            op, src, rnd, rev, arg, pad, a, sv = _INS.unpack_from(plan, blob_off + off_ins + i * _INS.size)
            ins.append((op, src, arg))
        stages.append(Stage(tasks, views, ins, n_items))
    return stages


# ----------------------------------------------------------- access sets --

@dataclass
class Access:
    """Elements of one view an item touches: `coords` is a list of index
    arrays (one per iteration dim, broadcastable) or a flat element array."""
    space: int
    write: bool
    item: tuple          # (stage, task, item) identity
    what: str
    lo: int = 0
    hi: int = 0
    _addr: object = field(default=None, repr=False)
    _gen: object = field(default=None, repr=False)
    # for a view whose element addresses are one-to-one with its coordinates:
    # (offset, strides, dtype) and the coordinate box [(a, b)] it covers
    geom: object = None
    box: object = None

    def addresses(self) -> np.ndarray:
        if self._addr is None:
            self._addr = np.unique(self._gen())
        return self._addr


def _view_bytes(v: View, idx) -> np.ndarray:
    """Byte addresses of view elements at coordinates idx (broadcast arrays)."""
    e = np.int64(v.offset)
    for d, c in enumerate(idx):
        e = e + np.asarray(c, dtype=np.int64) * v.strides[d]
    es = ESIZE[v.dtype]
    e = np.asarray(e, dtype=np.int64).reshape(-1)
    if es == 1:
        return e
    return (e[:, None] * es + np.arange(es, dtype=np.int64)[None, :]).reshape(-1)


def _view_box(v: View, ranges) -> tuple:
    """Byte interval [lo, hi) bounding a view over coordinate ranges [(a, b)]."""
    lo = hi = v.offset
    for d, (a, b) in enumerate(ranges):
        if b <= a:
            return (0, 0)
        s = v.strides[d]
        x, y = a * s, (b - 1) * s
        lo += min(x, y)
        hi += max(x, y)
    es = ESIZE[v.dtype]
    return (lo * es, (hi + 1) * es)


def _one_to_one(strides, extents) -> bool:
    """Whether distinct coordinates within `extents` always address distinct
    elements: sorted by magnitude, each stride is nonzero and exceeds the span
    of all smaller ones."""
    pairs = sorted((abs(s), n) for s, n in zip(strides, extents) if n > 1)
    span = 0
    for s, n in pairs:
        if s == 0 or s <= span:
            return False
        span += s * (n - 1)
    return True


def _disjoint_boxes(a, b) -> bool:
    return any(x1 <= y0 or y1 <= x0 for (x0, x1), (y0, y1) in zip(a, b))


def _share(a: np.ndarray, b: np.ndarray) -> bool:
    """Whether two sorted unique address arrays have an element in common."""
    if a.size == 0 or b.size == 0 or a[-1] < b[0] or b[-1] < a[0]:
        return False
    if a.size > b.size:
        a, b = b, a
    i = np.searchsorted(b, a)
    i[i == b.size] = b.size - 1
    return bool((b[i] == a).any())


def _unravel(e: np.ndarray, dims, nd) -> list:
    c = []
    for d in range(nd - 1, 0, -1):
        c.append(e % dims[d])
        e = e // dims[d]
    c.append(e)
    c = c[::-1]
    return c + [np.zeros_like(e)] * (4 - len(c))


class Checker:
    """Races of a compiled program's plan (tk.Program or its plan bytes plus
    the program text)."""

    def __init__(self, program):
        text = program.text
        self.stages = decode(program.plan_bytes())
        self.n_in = sum(1 for l in text.splitlines() if l.split()[:1] == ["in"])
        self.n_out = sum(1 for l in text.splitlines() if l.split()[:1] == ["out"])
        self.inplace = {}
        for l in text.splitlines():
            t = l.split()
            if t[:1] == ["inplace"]:
                self.inplace[int(t[1])] = int(t[2])
        self.ws_base = self.n_in + self.n_out

    def space(self, base: int) -> int:
        """Memory identity of a base slot: an in-place output slot is its input."""
        if self.n_in <= base < self.n_in + self.n_out and (base - self.n_in) in self.inplace:
            return self.inplace[base - self.n_in]
        return base

    # -- per-item accesses ---------------------------------------------------
    def _prog_views(self, st: Stage, first: int, length: int):
        """(view index, is_write) of an expression program's view operands."""
        out = []
        for op, src, arg in st.ins[first:first + length]:
            if op == VM_STORE:
                out.append((arg, True))
            elif src == SRC_VIEW:
                out.append((arg, False))
        return out

    def _acc(self, out, st, vi, write, item, what, ranges, gen, extents=None):
        v = st.views[vi]
        lo, hi = _view_box(v, ranges)
        if hi <= lo:
            return
        a = Access(self.space(v.base), write, item, what, lo, hi, _gen=gen)
        if extents is not None and _one_to_one(v.strides[:len(extents)], extents):
            a.geom = (v.offset, v.strides[:len(extents)], v.dtype)
            a.box = tuple(ranges)
        out.append(a)

    def _scratch(self, out, item, what, write, byte_lo, idx_fn):
        """fp32 partials in the workspace at byte offset byte_lo + 4 * idx."""
        def gen():
            e = np.asarray(idx_fn(), dtype=np.int64).reshape(-1)
            return (byte_lo + 4 * e[:, None] + np.arange(4, dtype=np.int64)[None, :]).reshape(-1)
        a = gen()
        if a.size:
            out.append(Access(self.ws_base, write, item, what, int(a.min()), int(a.max()) + 1, _addr=np.unique(a)))

    def _grid_views(self, out, st, t, item, views, r0, r1, c0, c1, what):
        """Epilogue views over outputs rows [r0, r1) x cols [c0, c1) of a
        product's [m, n] iteration space (output (r, c) is element r * n + c
        of the task's iteration dims)."""
        if t.ndim == 2 and t.dims[0] == t.m and t.dims[1] == t.n:
            for vi, w in views:
                v = st.views[vi]
                rr, cc = np.arange(r0, r1), np.arange(c0, c1)
                self._acc(out, st, vi, w, item, what, [(r0, r1), (c0, c1)],
                          lambda v=v, rr=rr, cc=cc: _view_bytes(v, (rr[:, None], cc[None, :])),
                          extents=(t.m, t.n))
            return
        for r in range(r0, r1):  # collapsed iteration space: row by row
            self._linear_views(out, st, t, item, views, r * t.n + c0, r * t.n + c1, t.dims, max(1, t.ndim), what)

    def _linear_views(self, out, st, t, item, views, e0, e1, dims, nd, what):
        """Views over linear elements [e0, e1) of an iteration space."""
        if e1 <= e0:
            return
        for vi, w in views:
            v = st.views[vi]

            def gen(v=v):
                e = np.arange(e0, e1, dtype=np.int64)
                return _view_bytes(v, _unravel(e, dims, nd))
            # bounding box of the coordinates the linear range reaches
            first = _unravel(np.array([e0]), dims, nd)
            last = _unravel(np.array([e1 - 1]), dims, nd)
            ranges = []
            spans_more = False
            for d in range(4):
                a, b = int(first[d][0]), int(last[d][0])
                if spans_more or d >= nd:
                    ranges.append((0, dims[d] if d < nd else 1))
                    continue
                if a == b:
                    ranges.append((a, a + 1))
                else:
                    ranges.append((min(a, b), max(a, b) + 1))
                    spans_more = True
            self._acc(out, st, vi, w, item, what, ranges, gen)

    def item_accesses(self, s: int, st: Stage) -> list:
        out = []
        for ti, t in enumerate(st.tasks):
            epi = self._prog_views(st, t.expr_first, t.expr_len)
            fin = self._prog_views(st, t.fin_first, t.fin_len)
            bsum = self._prog_views(st, t.bs_first, t.bs_len)
            name = f"stage {s} task {ti} kind {t.kind}"
            if t.kind in (T_GEMM_MFMA, T_GEMM_SIMT):
                bm = 128 if (t.kind == T_GEMM_MFMA and t.tile == 0) else 64
                tiles = t.tiles_m * t.tiles_n
                for it in range(t.n_items):
                    sp, tile = it // tiles, it % tiles
                    tm, tn = tile // t.tiles_n, tile % t.tiles_n
                    m0, n0 = tm * bm, tn * bm
                    m1, n1 = min(m0 + bm, t.m), min(n0 + bm, t.n)
                    kb = sp * t.kchunk
                    ke = min(kb + t.kchunk, t.k)
                    item = (s, ti, it)
                    A, B = st.views[t.va], st.views[t.vb]
                    kk = np.arange(kb, ke)
                    rr, cc = np.arange(m0, m1), np.arange(n0, n1)
                    # A's element (m, k) at stride[0], stride[1]; B's (n, k) at k * stride[0] + n * stride[1]
                    self._acc(out, st, t.va, False, item, name + " A", [(m0, m1), (kb, ke)],
                              lambda A=A, rr=rr, kk=kk: _view_bytes(A, (rr[:, None], kk[None, :])))
                    self._acc(out, st, t.vb, False, item, name + " B", [(kb, ke), (n0, n1)],
                              lambda B=B, kk=kk, cc=cc: _view_bytes(B, (kk[:, None], cc[None, :])))
                    if t.flags & F_PARTIAL:
                        mm, nn = t.m, t.n
                        self._scratch(out, item, name + " partial", True, t.scratch,
                                      lambda sp=sp, rr=rr, cc=cc, mm=mm, nn=nn:
                                      sp * mm * nn + rr[:, None] * nn + cc[None, :])
                    else:
                        self._grid_views(out, st, t, item, epi, m0, m1, n0, n1, name + " epilogue")
                    if t.flags & F_BSUM and tm == 0:
                        # the first tile row also sums B over all of K for its
                        # columns and runs the fused reduction's finish on them
                        kall = np.arange(0, t.k)
                        self._acc(out, st, t.vb, False, item, name + " B column sums", [(0, t.k), (n0, n1)],
                                  lambda B=B, kall=kall, cc=cc: _view_bytes(B, (kall[:, None], cc[None, :])))
                        self._linear_views(out, st, t, item, bsum, n0, n1, (t.n, 1, 1, 1), 1,
                                           name + " column sums")
            elif t.kind == T_GEMM_REDUCE:
                total = t.m * t.n
                for it in range(t.n_items):
                    e0, e1 = it * 4096, min((it + 1) * 4096, total)
                    item = (s, ti, it)
                    self._scratch(out, item, name + " partials", False, t.scratch,
                                  lambda e0=e0, e1=e1, total=total, sp=t.split:
                                  (np.arange(sp)[:, None] * total + np.arange(e0, e1)[None, :]))
                    self._linear_views(out, st, t, item, epi, e0, e1, (t.m, t.n, 1, 1), 2, name + " epilogue")
            elif t.kind == T_GEMV_Q8:
                X, Q, S = st.views[t.va], st.views[t.vb], st.views[t.vs]
                nb = (t.k + 31) // 32
                for it in range(t.n_items):
                    cb, r0 = it % t.tiles_n, (it // t.tiles_n) * GEMV_ROWS
                    r1 = min(r0 + GEMV_ROWS, t.m)
                    c0, c1 = cb * 16, min(cb * 16 + 16, t.n)
                    item = (s, ti, it)
                    rr, cc, kk = np.arange(r0, r1), np.arange(c0, c1), np.arange(t.k)
                    self._acc(out, st, t.va, False, item, name + " x", [(r0, r1), (0, t.k)],
                              lambda X=X, rr=rr, kk=kk: _view_bytes(X, (rr[:, None], kk[None, :])))
                    self._acc(out, st, t.vb, False, item, name + " q", [(c0, c1), (0, t.k)],
                              lambda Q=Q, cc=cc, kk=kk: _view_bytes(Q, (cc[:, None], kk[None, :])))
                    self._acc(out, st, t.vs, False, item, name + " s", [(c0, c1), (0, nb)],
                              lambda S=S, cc=cc, nb=nb: _view_bytes(S, (cc[:, None], np.arange(nb)[None, :])))
                    self._grid_views(out, st, t, item, epi, r0, r1, c0, c1, name + " epilogue")
            elif t.kind == T_EW:
                numel = int(np.prod(t.dims))
                for it in range(t.n_items):
                    self._linear_views(out, st, t, (s, ti, it), epi, it * 4096, min((it + 1) * 4096, numel),
                                       t.dims, max(1, t.ndim), name)
            elif t.kind == T_RED_ROWS:
                R = t.k
                for it in range(t.n_items):
                    row, part = it // t.split, it % t.split
                    kb = part * t.kchunk
                    ke = min(kb + t.kchunk, R)
                    item = (s, ti, it)
                    self._linear_views(out, st, t, item, epi, row * R + kb, row * R + ke, t.dims,
                                       max(1, t.ndim), name + " source")
                    if t.flags & F_PARTIAL:
                        self._scratch(out, item, name + " partial", True, t.scratch,
                                      lambda row=row, part=part, sp=t.split: np.array([row * sp + part]))
                    else:
                        self._linear_views(out, st, t, item, fin, row, row + 1, (t.m, 1, 1, 1), 1, name + " finish")
            elif t.kind == T_RED_COLS:
                W = 8 if t.width == 8 else 1
                per = 64 if t.flags & F_COLLANES32 else 32 * W  # columns per item
                cols, R = t.m, t.k
                for it in range(t.n_items):
                    cb, part = it // t.split, it % t.split
                    c0, c1 = cb * per, min(cb * per + per, cols)
                    rb = part * t.kchunk
                    re_ = min(rb + t.kchunk, R)
                    item = (s, ti, it)
                    if c1 <= c0 or re_ <= rb:
                        continue
                    # source elements r * cols + c of the iteration space
                    for vi, w in epi:
                        v = st.views[vi]

                        def gen(v=v, c0=c0, c1=c1, rb=rb, re_=re_):
                            e = (np.arange(rb, re_)[:, None] * cols + np.arange(c0, c1)[None, :]).reshape(-1)
                            return _view_bytes(v, _unravel(e, t.dims, max(1, t.ndim)))
                        a = gen()
                        out.append(Access(self.space(v.base), w, item, name + " source", int(a.min()),
                                          int(a.max()) + 1, _addr=np.unique(a)))
                    if t.flags & F_PARTIAL:
                        self._scratch(out, item, name + " partial", True, t.scratch,
                                      lambda part=part, c0=c0, c1=c1: part * cols + np.arange(c0, c1))
                    else:
                        self._linear_views(out, st, t, item, fin, c0, c1, (t.m, 1, 1, 1), 1, name + " finish")
            elif t.kind == T_RED_FINAL:
                cols_layout = (t.tile & 1) != 0
                for it in range(t.n_items):
                    rows = np.array([it]) if t.flags & F_ROWWG else np.arange(it * KBLOCK, min((it + 1) * KBLOCK, t.m))
                    if rows.size == 0:
                        continue
                    item = (s, ti, it)
                    if cols_layout:
                        idx = lambda rows=rows: np.arange(t.split)[:, None] * t.m + rows[None, :]
                    else:
                        idx = lambda rows=rows: rows[:, None] * t.split + np.arange(t.split)[None, :]
                    self._scratch(out, item, name + " partials", False, t.scratch, idx)
                    self._linear_views(out, st, t, item, fin, int(rows[0]), int(rows[-1]) + 1, (t.m, 1, 1, 1), 1,
                                       name + " finish")
            else:
                raise NotImplementedError(f"race checker: task kind {t.kind}")
        return out

    # -- checking ------------------------------------------------------------
    def races(self, merge=(), first_only: bool = False) -> list:
        """Conflicting accesses per (merged) stage.  `merge` lists stage
        indices s whose barrier to stage s + 1 is dropped; `first_only`
        stops at the first race found."""
        groups, cur = [], [0]
        for s in range(1, len(self.stages)):
            if (s - 1) in set(merge):
                cur.append(s)
            else:
                groups.append(cur)
                cur = [s]
        groups.append(cur)
        found = []
        for g in groups:
            acc = []
            for s in g:
                acc += self.item_accesses(s, self.stages[s])
            found += self._conflicts(acc, first_only)
            if found and first_only:
                break
        return found

    @staticmethod
    def _conflicts(acc, first_only=False) -> list:
        found = []
        by_space = {}
        for a in acc:
            by_space.setdefault(a.space, []).append(a)
        for space, lst in by_space.items():
            writes = [a for a in lst if a.write]
            if not writes:
                continue
            lo = np.array([a.lo for a in lst], dtype=np.int64)
            hi = np.array([a.hi for a in lst], dtype=np.int64)
            order = np.argsort(lo, kind="stable")
            slo = lo[order]
            for w in writes:
                # candidates: intervals starting before w ends and ending after w starts
                n = int(np.searchsorted(slo, w.hi, side="left"))
                cand = order[:n]
                cand = cand[hi[cand] > w.lo]
                for ci in cand:
                    o = lst[int(ci)]
                    if o is w or o.item == w.item:
                        continue
                    if o.write and id(o) < id(w):
                        continue  # each write/write pair once
                    if (w.geom is not None and w.geom == o.geom and len(w.box) == len(o.box)
                            and _disjoint_boxes(w.box, o.box)):
                        continue  # one view, one-to-one, disjoint coordinates
                    if _share(w.addresses(), o.addresses()):
                        found.append((w.item, w.what, o.item, o.what, "write/write" if o.write else "write/read"))
                        if first_only:
                            return found
        return found


def check(program, merge=(), first_only: bool = False) -> list:
    """Races in `program`'s plan (an empty list when the schedule is safe)."""
    return Checker(program).races(merge, first_only)


def needed_barriers(program) -> list:
    """For each barrier (between stages s and s + 1): whether dropping it
    alone makes the schedule race."""
    c = Checker(program)
    return [bool(c.races(merge=[s], first_only=True)) for s in range(len(c.stages) - 1)]
