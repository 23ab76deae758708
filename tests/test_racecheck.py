"""The schedule race checker (persistent_whole_step_amd.racecheck) on the CPU.

Every plan the workloads compile to is race-free (no item of a stage writes
bytes another item of that stage reads or writes), and every grid barrier in
them is needed: dropping any one of them (merging two stages) makes the
checker report a race.  Planted mistakes in a plan's descriptors are caught.
"""
import copy

import pytest

from persistent_whole_step_amd import programs, racecheck, tk
from persistent_whole_step_amd.programs import Program

SMALL = {
    "c2s": dict(kind="mlp", dims=(192, 320, 256, 48), batch=96, dtype="bf16", lr=1e-3),
    "c3r": dict(kind="gemv", k=1024, n=1024, layers=3, rows=6),
    "c4s": dict(kind="mlp", dims=(256, 384, 256, 128), batch=160, dtype="bf16", lr=1e-4),
    "c5s": dict(kind="residual", width=256, layers=4, batch=96, dtype="f16", lr=1e-4),
    "c2sa": dict(kind="mlp", dims=(192, 320, 256, 48), batch=96, dtype="bf16", lr=1e-3,
                 optimizer=programs.AdamW(), adam_t=5),
    "c5sa": dict(kind="residual", width=256, layers=4, batch=96, dtype="f16", lr=1e-4,
                 optimizer=programs.AdamW(weight_decay=0.1), adam_t=2),
}


def _plan(cfg, **opts):
    return tk.compile(programs.build(cfg).text(), device=-1, **opts)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_plans_are_race_free(name):
    assert racecheck.check(_plan(programs.CONFIGS[name])) == []


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("opts", [{}, {"barrier_every_op": 1}, {"batch_epilogues": 1}, {"gemm_tile": 2}])
def test_small_plans_are_race_free(name, opts):
    assert racecheck.check(_plan(SMALL[name], **opts)) == []


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_every_barrier_is_needed(name):
    need = racecheck.needed_barriers(_plan(programs.CONFIGS[name]))
    assert need and all(need), need


@pytest.mark.parametrize("name", ["c5s", "c2sa", "c4s"])
def test_every_barrier_is_needed_small(name):
    need = racecheck.needed_barriers(_plan(SMALL[name]))
    assert need and all(need), need


@pytest.mark.parametrize("split", [2, 4])
def test_split_k_plan_is_race_free(split):
    p = Program()
    a = p.input("a", "bf16", (256, 2048))
    b = p.input("b", "bf16", (2048, 384))
    bias = p.input("bias", "bf16", (384,))
    y = p.op("addmm", [bias, a, b], "bf16", (256, 384))
    p.output(p.op("relu", [y], "bf16"))
    prog = tk.compile(p.text(), device=-1, gemm_split_k=split)
    assert racecheck.check(prog) == []
    assert all(racecheck.needed_barriers(prog))


def test_staged_commit_plan_is_race_free_and_its_commit_barrier_needed():
    p = Program()
    a = p.input("a", "bf16", (192, 192))
    W = p.input("W", "bf16", (192, 192))
    g = p.op("mm", [a, W], "bf16", (192, 192))
    p.output(p.op("sub", [W, g], "bf16", alpha=0.5), inplace_of=W)
    prog = tk.compile(p.text(), device=-1)
    assert prog.query()["staged_commits"] == 1
    assert racecheck.check(prog) == []
    # committing in the tile's own stage would overwrite W while other tiles read it
    assert racecheck.needed_barriers(prog) == [True]


def _planted(prog, mutate):
    c = racecheck.Checker(prog)
    c.stages = copy.deepcopy(c.stages)
    mutate(c.stages)
    return c.races(first_only=True)


def test_planted_overlapping_store_is_caught():
    """A contraction tile's store view moved onto the operand that the
    stage's tiles read: the checker reports it."""
    prog = _plan(SMALL["c2s"])

    def mutate(stages):
        for st in stages:
            for t in st.tasks:
                if t.kind == racecheck.T_GEMM_MFMA:
                    stores = [arg for op, src, arg in st.ins[t.expr_first:t.expr_first + t.expr_len]
                              if op == racecheck.VM_STORE]
                    a = st.views[t.va]
                    st.views[stores[0]] = racecheck.View(a.offset, (a.strides[0], a.strides[1], 0, 0), a.base,
                                                         st.views[stores[0]].dtype)
                    return
    assert _planted(prog, mutate)


def test_planted_wrong_tile_count_is_caught():
    """Two items of one elementwise task addressing the same elements (an
    item count past the iteration space after a shape mix-up) race."""
    p = Program()
    x = p.input("x", "f32", (64, 200))
    p.output(p.op("mul", [x, 2.0], "f32"))
    prog = tk.compile(p.text(), device=-1, fuse_pointwise=0)
    assert racecheck.check(prog) == []

    def mutate(stages):
        for st in stages:
            for t in st.tasks:
                if t.kind == racecheck.T_EW:
                    t.dims = (t.dims[0] * 2,) + tuple(t.dims[1:])
                    t.n_items *= 2
                    # the store view wraps around: a stride that folds the doubled space onto itself
                    for op, src, arg in st.ins[t.expr_first:t.expr_first + t.expr_len]:
                        if op == racecheck.VM_STORE:
                            v = st.views[arg]
                            n = int(t.dims[0] // 2)
                            st.views[arg] = racecheck.View(v.offset, tuple(s if i else 0 for i, s in
                                                                           enumerate(v.strides)), v.base, v.dtype)
                    return
    assert _planted(prog, mutate)
