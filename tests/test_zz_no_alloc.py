"""The allocation-free entry point (tk_run_into_noalloc) against tk_run_into.

The no-alloc call runs the same kernel and plan in the library's static
per-device workspace, so its outputs must equal tk_run_into's bit for bit.
Two calls in a row, the second with a smaller program, check that each call
starts from a cleared workspace header; a program whose workspace exceeds the
static workspace is rejected before anything runs.
"""
import ctypes
import sys

import numpy as np
import pytest

from persistent_whole_step_amd import programs, tk
from persistent_whole_step_amd.programs import Program

from . import parity


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def test_noalloc_rejects_a_workspace_beyond_the_static_one():
    """A plan-only program whose arena exceeds 128 MiB: TK_E_WORKSPACE, with
    no device touched (the size is checked first)."""
    p = Program()
    x = p.input("x", "f32", (64, 1 << 20))
    y = p.op("mul", [x, 2.0], "f32")
    p.output(p.op("add", [y, y], "f32"))
    prog = tk.compile(p.text(), device=-1, fuse_pointwise=0)
    assert prog.query()["workspace_bytes"] > (128 << 20)
    ins = (tk.TkTensor * 1)()
    outs = (tk.TkTensor * 1)()
    rc = tk.lib().tk_run_into_noalloc(prog._h, ins, 1, outs, 1, None)
    assert tk.STATUS[rc] == "TK_E_WORKSPACE"
    assert b"static workspace" in tk.lib().tk_last_error()


def _run_both(name, cfg, seed):
    """tk_run_into (allocated workspace) and tk_run_into_noalloc on the same
    inputs; returns both output lists as host storage arrays."""
    import torch
    say("no-alloc vs run_into", name)
    prog = programs.build(cfg)
    p = tk.compile(prog.text(), device=0, launch_mode=1)
    ins = programs.inputs_for(cfg, seed)
    ref, _ = parity.gpu_run(prog, [a.copy() for a in ins], launch_mode=1)
    tins = [parity.to_torch(a.copy(), s.dtype) for a, s in zip(ins, prog.inputs)]
    inplace = p._inplace_map()
    outs = []
    for slot, s in enumerate(prog.outputs):
        if slot in inplace:
            outs.append(tins[inplace[slot]])
        else:
            outs.append(torch.full(s.shape, float("nan"), dtype=parity.torch_dtype(s.dtype), device="cuda:0"))
    p.run_into_noalloc(*tins, outputs=outs)
    torch.cuda.synchronize()
    got = [parity.to_numpy(o, s.dtype) for o, s in zip(outs, prog.outputs)]
    return prog, ref, got


@pytest.mark.gpu
def test_noalloc_matches_run_into_twice_then_smaller():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [("c2s", dict(kind="mlp", dims=(192, 320, 256, 48), batch=96, dtype="bf16", lr=1e-3), 1),
             ("c1", dict(programs.CONFIGS["c1"]), 2)]
    for name, cfg, seed in cases:
        prog, ref, got = _run_both(name, cfg, seed)
        for g, r, s in zip(got, ref, prog.outputs):
            parity.assert_bitexact(g, r, s.dtype, f"{name} {s.buf}")
