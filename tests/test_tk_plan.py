"""CPU tests of libtk without a GPU: the C ABI loads and exports every symbol
include/tk.h declares; plan-only compiles of every workload; the scheduler's
fusion/inlining/in-place decisions (trainkernel codegen.py `_Generator`);
compile-time rejections; and the run-time buffer checks of tk_validate_into
(runtime.py `run_into`) on descriptors that are never dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

from persistent_whole_step_amd import programs, tk
from persistent_whole_step_amd.programs import Program

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "tk.h")).read()
    return sorted(set(re.findall(r"\b(tk_[a-z_]+)\s*\(", text)) - {"tk_alloc_fn"})


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tk.LIB_PATH)
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_plan_only_compile_of_workloads(name):
    p = programs.build(programs.CONFIGS[name])
    prog = tk.compile(p.text(), device=-1)
    q = prog.query()
    assert q["grid_barriers"] == q["n_stages"] - 1
    assert q["workspace_bytes"] >= 16384
    assert q["grid_size"] >= 1 and q["grid_size"] <= 256
    n_params = sum(1 for k, _ in p.inplace.items())
    assert q["direct_state_commits"] == n_params
    assert "stage 0:" in prog.dump()


@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c5"])
def test_plan_only_compile_with_adamw(name):
    cfg = dict(programs.CONFIGS[name], optimizer=programs.AdamW())
    p = programs.build(cfg)
    q = tk.compile(p.text(), device=-1).query()
    # parameter, first and second moment of every parameter committed in place
    assert len(p.inplace) == len(p.inputs) - 4  # inputs: x, t, params, (m, v) per param, c1, c2
    assert q["direct_state_commits"] == len(p.inplace)
    assert q["staged_commits"] == 0
    assert q["grid_barriers"] == q["n_stages"] - 1


def test_mlp_schedule_decisions():
    p = programs.build(programs.CONFIGS["c1"])
    q = tk.compile(p.text(), device=-1).query()
    # gm + threshold_backward chain: one epilogue fusion; the first layer's
    # relu is written by its addmm tile (side program: both the
    # pre-activation and the activation are read later); the output layer's
    # tile also computes d, d^2 and the loss gradient (a chain extended by
    # its further descendants); every weight update folds into its gradient
    # tile and every bias update into the finishing program of its batch sum
    assert q["fused_epilogues"] == 1
    assert q["side_epilogues"] == 2
    assert q["fused_updates"] == 4
    assert q["inlined_ops"] == 0
    assert q["n_stages"] == 4


def test_adamw_update_folds_like_sgd():
    # the whole AdamW update (two states and the parameter, all in place) is
    # evaluated by the gradient's tile or the bias sum's finishing program:
    # the step keeps SGD's stage count
    for name in ("c1", "c2"):
        sgd = tk.compile(programs.build(programs.CONFIGS[name]).text(), device=-1).query()
        p = programs.build(dict(programs.CONFIGS[name], optimizer=programs.AdamW()))
        q = tk.compile(p.text(), device=-1).query()
        assert q["n_stages"] == sgd["n_stages"]
        assert q["fused_updates"] == len(p.inplace) == 3 * sgd["fused_updates"]
        assert q["materialized_ops"] == sgd["materialized_ops"]


def _gemv_program(scale_kind: str):
    p = Program()
    x = p.input("x", "bf16", (1, 256))
    q = p.input("q", "i8", (64, 256))
    s = p.input("s", "f32", (64, 8))
    b = p.input("b", "f32", (64,))
    h = p.op("addmm_q8", [b, x, q, s], "bf16", (1, 64))
    if scale_kind == "computed":
        s2 = p.op("mul", [s, 2.0], "f32")
        p.output(p.op("addmm_q8", [b, x, q, s2], "bf16", (1, 64)))
    elif scale_kind == "updated":
        p.output(p.op("addmm_q8", [b, x, q, s], "bf16", (1, 64)))
        p.output(p.op("mul", [s, 0.5], "f32"), inplace_of=s)
    p.output(h)
    return p


@pytest.mark.parametrize("kind", ["input", "computed", "updated"])
def test_gemv_scale_sources(kind):
    # scales that are inputs, computed values or updated in place all plan as
    # two int8 products; an in-place update of the scales waits for them
    p = _gemv_program(kind)
    if kind == "input":
        p.output(p.op("addmm_q8", [p.inputs[3], p.inputs[0], p.inputs[1], p.inputs[2]], "bf16", (1, 64)))
    prog = tk.compile(p.text(), device=-1)
    d = prog.dump()
    assert sum(line.strip().startswith("gemv_q8") for line in d.splitlines()) == 2
    if kind == "updated":
        # both products read s in stage 0; the direct update of s runs after
        stages = d.split("stage ")[1:]
        assert "gemv_q8" in stages[0] and "gemv_q8" not in stages[1] and "ew items=1 : mul" in stages[1]
        assert prog.query()["direct_state_commits"] == 1


def test_activation_quantisation_flag():
    # xq on a q8 product reaches its GEMV task; it is refused elsewhere and
    # for values other than 0 and 1
    d = tk.compile(programs.gemv_q8_stack(256, 256, 2, xq=True).text(), device=-1).dump()
    assert d.count("[activations quantised to Q8_0]") == 2
    d = tk.compile(programs.gemv_q8_stack(256, 256, 2).text(), device=-1).dump()
    assert "quantised" not in d
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (3, 4))
    p.output(p.op("mm", [a, b], "f32", (2, 4), xq=1.0))
    with pytest.raises(tk.TkError, match="xq"):
        tk.compile(p.text(), device=-1)
    p = Program()
    x = p.input("x", "bf16", (1, 64))
    q = p.input("q", "i8", (8, 64))
    s = p.input("s", "f32", (8, 2))
    p.output(p.op("mm_q8", [x, q, s], "f32", (1, 8), xq=2.0))
    with pytest.raises(tk.TkError, match="xq"):
        tk.compile(p.text(), device=-1)


def _tile_update(later_read: bool):
    p = Program()
    a = p.input("a", "f32", (8, 8))
    b = p.input("b", "f32", (8, 8))
    W = p.input("W", "f32", (8, 8))
    g = p.op("mm", [a, b], "f32", (8, 8))
    Wn = p.op("sub", [W, g], "f32", alpha=0.5)
    if later_read:
        # reads the old W after the update in program order, from the same tile
        y = p.op("mul", [W, g], "f32")
        p.output(y)
    p.output(Wn, inplace_of=W)
    return p


def test_tile_update_commits_directly():
    q = tk.compile(_tile_update(False).text(), device=-1).query()
    assert q["direct_state_commits"] == 1 and q["fused_updates"] == 1 and q["n_stages"] == 1


def test_tile_update_staged_when_tile_reads_target_after_store():
    q = tk.compile(_tile_update(True).text(), device=-1).query()
    assert q["direct_state_commits"] == 0 and q["staged_commits"] == 1


def test_tile_update_staged_when_contraction_reads_target():
    # the tile's own operand is the target: the update cannot overwrite it
    p = Program()
    a = p.input("a", "f32", (8, 8))
    W = p.input("W", "f32", (8, 8))
    g = p.op("mm", [a, W], "f32", (8, 8))
    p.output(p.op("sub", [W, g], "f32", alpha=0.5), inplace_of=W)
    q = tk.compile(p.text(), device=-1).query()
    assert q["direct_state_commits"] == 0 and q["staged_commits"] == 1


def test_side_epilogue_stores_values_read_later():
    # h = a@b is read later (by threshold_backward) and so is r = relu(h): the
    # tile writes both, and no separate pointwise stage remains
    p = Program()
    a = p.input("a", "f32", (8, 8))
    b = p.input("b", "f32", (8, 8))
    g = p.input("g", "f32", (8, 8))
    h = p.op("mm", [a, b], "f32", (8, 8))
    r = p.op("relu", [h], "f32")
    m = p.op("mm", [r, b], "f32", (8, 8))
    t = p.op("threshold_backward", [g, h], "f32", threshold=0.0)
    p.output(m)
    p.output(t)
    q = tk.compile(p.text(), device=-1).query()
    assert q["side_epilogues"] == 1
    assert q["n_stages"] == 2


def test_fusion_stops_at_returned_values():
    # pass 1 never fuses a chain whose link is a returned value
    p = Program()
    a = p.input("a", "f32", (8, 8))
    b = p.input("b", "f32", (8, 8))
    y = p.op("mm", [a, b], "f32", (8, 8))
    z = p.op("relu", [y], "f32")
    p.output(z)
    q = tk.compile(p.text(), device=-1).query()
    # relu output returned: pass 2 writes it from the tile instead (root discarded)
    assert q["fused_epilogues"] == 0 and q["side_epilogues"] == 1 and q["n_stages"] == 1


def test_non_identity_view_blocks_fusion():
    p = Program()
    a = p.input("a", "f32", (8, 8))
    b = p.input("b", "f32", (8, 8))
    y = p.op("mm", [a, b], "f32", (8, 8))
    z = p.op("relu", [y.T], "f32", shape=(8, 8))   # transposed read of the root
    w = p.op("mul", [z, 2.0], "f32")
    p.output(w)
    q = tk.compile(p.text(), device=-1).query()
    assert q["fused_epilogues"] == 0 and q["n_stages"] >= 2


def test_fusion_disabled_by_options():
    p = programs.build(programs.CONFIGS["c1"])
    q = tk.compile(p.text(), device=-1, fuse_epilogues=0, fuse_pointwise=0).query()
    assert q["fused_epilogues"] == 0 and q["fused_updates"] == 0 and q["inlined_ops"] == 0
    q2 = tk.compile(p.text(), device=-1, barrier_every_op=1).query()
    assert q2["n_stages"] >= q2["materialized_ops"]


def test_direct_commit_refused_when_target_read_later():
    # W read by an op after the update: the update must be staged and committed last
    p = Program()
    W = p.input("W", "f32", (4, 4))
    g = p.input("g", "f32", (4, 4))
    Wn = p.op("sub", [W, g], "f32", alpha=0.5)
    later = p.op("mul", [W, 2.0], "f32")
    p.output(Wn, inplace_of=W)
    p.output(later)
    q = tk.compile(p.text(), device=-1).query()
    assert q["direct_state_commits"] == 0 and q["staged_commits"] == 1


@pytest.mark.parametrize("mutate,code", [
    (lambda t: t.replace("#0x1.0000000000000p+1", "#inf"), "TK_E_ARG"),
    (lambda t: t.replace(" mul ", " tanh "), "TK_E_UNSUPPORTED"),
    (lambda t: t.replace("tkir 1", "tkir 9"), "TK_E_PARSE"),
    (lambda t: t.replace("y:f32:4:1:0", "y:f32:4:2:0"), "TK_E_STRIDE"),
    (lambda t: t + "junk", "TK_E_PARSE"),
])
def test_compile_rejections(mutate, code):
    p = Program()
    a = p.input("a", "f32", (4,))
    p.output(p.op("mul", [a, 2.0], "f32", name="y"))
    with pytest.raises(tk.TkError) as ei:
        tk.compile(mutate(p.text()), device=-1)
    assert ei.value.status_name == code


def test_compile_rejects_bad_shapes_and_inplace():
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (4,))
    p.output(p.op("add", [a, b], "f32"))
    with pytest.raises(tk.TkError, match="broadcast"):
        tk.compile(p.text(), device=-1)
    p = Program()
    a = p.input("a", "f32", (2, 3))
    b = p.input("b", "f32", (4, 2))
    p.output(p.op("mm", [a, b], "f32", (2, 2)))
    with pytest.raises(tk.TkError, match="compatible"):
        tk.compile(p.text(), device=-1)
    p = Program()
    a = p.input("a", "f32", (4,))
    c = p.input("c", "f32", (4,))
    y = p.op("mul", [a, 2.0], "f32")
    p.output(y, inplace_of=a)
    p.inplace[1] = 0
    p.output(p.op("mul", [c, 2.0], "f32"))
    with pytest.raises(tk.TkError, match="distinct"):
        tk.compile(p.text(), device=-1)
    p = Program()
    a = p.input("a", "f32", (4,))
    p.output(a)
    p.inplace[0] = 0
    with pytest.raises(tk.TkError, match="computed values"):
        tk.compile(p.text(), device=-1)


@pytest.mark.parametrize("opt,val", [("blocks_per_cu", 0), ("blocks_per_cu", 9), ("threads_per_block", 128),
                                     ("gemm_split_k", 3), ("max_blocks", -1)])
def test_option_ranges(opt, val):
    p = programs.build(programs.CONFIGS["c1"])
    with pytest.raises(tk.TkError):
        tk.compile(p.text(), device=-1, **{opt: val})


# ------------------------------------------------ run-time buffer checks --

def _sgd_prog():
    p = Program()
    W = p.input("W", "f32", (4, 4))
    g = p.input("g", "f32", (4, 4))
    Wn = p.op("sub", [W, g], "f32", alpha=0.5)
    p.output(Wn, inplace_of=W)
    p.output(p.op("mul", [g, 2.0], "bf16"))
    return p


class Fake:
    """Non-overlapping fake device addresses."""
    def __init__(self):
        self.next = 1 << 40

    def take(self, nbytes):
        a = self.next
        self.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return a


def _setup():
    p = _sgd_prog()
    prog = tk.compile(p.text(), device=-1)
    f = Fake()
    W = tk.describe_fake((4, 4), "f32", f.take(64))
    g = tk.describe_fake((4, 4), "f32", f.take(64))
    o0 = W
    o1 = tk.describe_fake((4, 4), "bf16", f.take(32))
    wsb = prog.query()["workspace_bytes"]
    ws = tk.describe_fake((wsb,), "i8", f.take(wsb))
    return prog, [W, g], [o0, o1], ws, f


def test_validate_accepts_good_buffers():
    prog, ins, outs, ws, _ = _setup()
    tk.validate_fake(prog, ins, outs, ws)


def _expect(prog, ins, outs, ws, code):
    with pytest.raises(tk.TkError) as ei:
        tk.validate_fake(prog, ins, outs, ws)
    assert ei.value.status_name == code, str(ei.value)


def test_validate_rejections():
    prog, ins, outs, ws, f = _setup()
    _expect(prog, ins[:1], outs, ws, "TK_E_COUNT")
    _expect(prog, ins, outs[:1], ws, "TK_E_COUNT")
    bad = tk.describe_fake((4, 4), "bf16", f.take(64))
    _expect(prog, [ins[0], bad], outs, ws, "TK_E_DTYPE")
    bad = tk.describe_fake((4, 5), "f32", f.take(80))
    _expect(prog, [ins[0], bad], outs, ws, "TK_E_SHAPE")
    bad = tk.describe_fake((4, 4), "f32", f.take(64), strides=(1, 4))
    _expect(prog, [ins[0], bad], outs, ws, "TK_E_STRIDE")
    bad = tk.describe_fake((4, 4), "bf16", f.take(64), strides=(1, 4))
    _expect(prog, ins, [outs[0], bad], ws, "TK_E_STRIDE")
    other = tk.describe_fake((4, 4), "f32", f.take(64), device=1)
    _expect(prog, [ins[0], other], outs, ws, "TK_E_DEVICE")
    small = tk.describe_fake((100,), "i8", f.take(100))
    _expect(prog, ins, outs, small, "TK_E_WORKSPACE")
    unaligned = tk.describe_fake((ws.shape[0],), "i8", f.take(ws.shape[0]) + 8)
    _expect(prog, ins, outs, unaligned, "TK_E_WORKSPACE")
    # in-place slot not bound to its input
    _expect(prog, ins, [tk.describe_fake((4, 4), "f32", f.take(64)), outs[1]], ws, "TK_E_ALIAS")
    # output overlapping an input / another output / the workspace
    _expect(prog, ins, [outs[0], tk.describe_fake((4, 4), "bf16", ins[1].data)], ws, "TK_E_ALIAS")
    _expect(prog, ins, [outs[0], tk.describe_fake((4, 4), "bf16", ws.data + 256)], ws, "TK_E_ALIAS")
    # in-place target sharing storage with another input
    shared = tk.describe_fake((4, 4), "f32", ins[0].data + 32, storage=(ins[0].data, 1024))
    tgt = tk.describe_fake((4, 4), "f32", ins[0].data, storage=(ins[0].data, 1024))
    _expect(prog, [tgt, shared], [tgt, outs[1]], ws, "TK_E_ALIAS")
    # requires_grad on an in-place target
    rg = tk.describe_fake((4, 4), "f32", ins[0].data)
    rg.requires_grad = 1
    _expect(prog, [rg, ins[1]], [rg, outs[1]], ws, "TK_E_ARG")


def test_run_refused_for_plan_only_program():
    prog, ins, outs, ws, _ = _setup()
    arr_in = tk._array(ins)
    arr_out = tk._array(outs)
    st = tk.lib().tk_run_into(prog._h, arr_in, 2, arr_out, 2, ctypes.byref(ws), None)
    assert tk.STATUS[st] == "TK_E_DEVICE"


@pytest.mark.parametrize("name,marked,gemms", [("c1", 3, 5), ("c2", 7, 8), ("c5", 46, 47)])
def test_register_epilogue_marking(name, marked, gemms):
    """Contraction tiles whose epilogue is short and simple (no slots, 2-D
    chunk-aligned views, at most three loaded views) are marked to run it
    from registers; C1's 10-wide outputs and the loss-head programs that save
    slots keep the batches.  batch_epilogues=1 turns the register path off."""
    text = programs.build(programs.CONFIGS[name]).text()
    d = tk.compile(text, device=-1).dump()
    assert d.count("gemm_") == gemms
    assert d.count("[register epilogue]") == marked
    d1 = tk.compile(text, device=-1, batch_epilogues=1).dump()
    assert d1.count("[register epilogue]") == 0 and d1.count("[rows summed directly]") == 0


def test_column_sums_in_weight_gradient_tiles_or_read_directly():
    """A bias-gradient sum whose own items would give some workgroups of its
    stage one more item than the rest runs inside the weight-gradient
    product that reads the same gradient (its first tile row sums B over K
    and runs the sum's finish, the bias update included): in the 16-layer
    residual MLP every stage is full, so all 16 sums move and the step needs
    32 stages; in the 4096-wide MLP (K = 1024, whole 64-deep slices) all
    three move.  Otherwise the sums stay column reductions read straight from
    memory: one part up to 256 rows (the 3-layer bf16 MLP, 6 stages), fp32
    partials and a combine at 512 rows, one 32-row-lane part of 64 columns
    per item from 513 to 1024 rows (the 4096-wide MLP unfused)."""
    c2 = programs.build(programs.CONFIGS["c2"]).text()
    c5 = programs.build(programs.CONFIGS["c5"]).text()
    d = tk.compile(c2, device=-1)
    text = d.dump()
    assert text.count("[rows summed directly]") == 3 and "+column sums of B: " not in text
    assert d.query()["n_stages"] == 6
    d5 = tk.compile(c5, device=-1)
    t5 = d5.dump()
    assert t5.count("+column sums of B: ") == 16 and "reduce_cols" not in t5 and d5.query()["n_stages"] == 32
    u5 = tk.compile(c5, device=-1, fuse_epilogues=0).dump()
    assert "reduce_final" in u5 and "[rows summed directly]" in u5 and "[16 partials]" in u5
    c4 = programs.build(programs.CONFIGS["c4"]).text()
    d4 = tk.compile(c4, device=-1).dump()
    assert d4.count("+column sums of B: ") == 3 and "reduce_cols" not in d4
    u4 = tk.compile(c4, device=-1, colsum_fusion=-1).dump()
    assert u4.count("[rows summed directly]") == 3 and "reduce_cols items=64 : gb1" in u4


def test_column_sum_fusion_option():
    """colsum_fusion = 1 moves every legal bias-gradient sum into its
    weight-gradient tiles (all three of the 3-layer bf16 MLP, where the
    default keeps them: they add no round of items), -1 none (the residual
    MLP's 16 stay reductions); other values are rejected."""
    c2 = programs.build(programs.CONFIGS["c2"]).text()
    c5 = programs.build(programs.CONFIGS["c5"]).text()
    d2 = tk.compile(c2, device=-1, colsum_fusion=1).dump()
    assert d2.count("+column sums of B: ") == 3 and "reduce_cols" not in d2
    d5 = tk.compile(c5, device=-1, colsum_fusion=-1).dump()
    assert "+column sums of B: " not in d5 and d5.count("reduce_cols") == 16
    for bad in (2, -2):
        with pytest.raises(tk.TkError, match="colsum_fusion"):
            tk.compile(c5, device=-1, colsum_fusion=bad)
