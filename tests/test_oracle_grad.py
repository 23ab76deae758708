"""Pins for the oracle on whole training steps: the explicit backward graphs
(written out op by op, as the trainkernel README's supported subset requires:
"explicit differentiation" in a pure functional step) against central finite
differences in binary64, a hand-derived step, SGD closed forms and invariants
(transactional in-place commit, probe == base, ReLU masking).
"""
import os

import numpy as np
import pytest

from persistent_whole_step_amd import programs, synth
from persistent_whole_step_amd.programs import Program

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _loss_and_grads64(oracle_mod, prog, inputs):
    outs = oracle_mod.run64(prog.text(), inputs)
    return outs


def _fd_check(oracle_mod, prog_grads, prog_loss, inputs, param_idx, grad_slots, h=1e-5, tol=1e-6):
    outs = oracle_mod.run64(prog_grads.text(), inputs)
    for pi, gslot in zip(param_idx, grad_slots):
        g = outs[gslot]
        fd = np.zeros_like(g)
        base = inputs[pi]
        for idx in np.ndindex(base.shape):
            plus = [a.copy() for a in inputs]
            minus = [a.copy() for a in inputs]
            plus[pi][idx] += h
            minus[pi][idx] -= h
            lp = oracle_mod.run64(prog_loss.text(), plus)[0]
            lm = oracle_mod.run64(prog_loss.text(), minus)[0]
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1e-3, float(np.abs(g).max()))
        err = float(np.abs(fd - g).max()) / scale
        assert err <= tol, (pi, err)


def _preacts_away_from_kinks(oracle_mod, prog, inputs, margin=1e-3):
    probe = prog.probe()
    outs = oracle_mod.run64(probe.text(), inputs)
    names = [o.buf for o in probe.outputs]
    for name, v in zip(names, outs):
        if name.startswith("h") or name.startswith("z"):
            assert np.all(np.abs(v) > margin), f"{name} too close to the ReLU kink"


def test_mlp_gradients_match_finite_differences(oracle_mod):
    dims, batch = (4, 5, 2), 3
    prog_g = programs.mlp_step(dims, batch, "f32", lr=0.0, return_grads=True)
    prog_l = programs.mlp_step(dims, batch, "f32", lr=0.0)
    ins = [a.astype(np.float64) for a in synth.mlp_inputs(11, dims, batch, "f32")]
    _preacts_away_from_kinks(oracle_mod, prog_l, ins)
    # outputs: loss, W1', b1', W2', b2', gW1, gb1, gW2, gb2
    _fd_check(oracle_mod, prog_g, prog_l, ins, param_idx=[2, 3, 4, 5], grad_slots=[5, 6, 7, 8])


def test_three_layer_mlp_gradients(oracle_mod):
    dims, batch = (3, 4, 4, 2), 2
    prog_g = programs.mlp_step(dims, batch, "f32", lr=0.0, return_grads=True)
    prog_l = programs.mlp_step(dims, batch, "f32", lr=0.0)
    ins = [a.astype(np.float64) for a in synth.mlp_inputs(5, dims, batch, "f32")]
    _preacts_away_from_kinks(oracle_mod, prog_l, ins)
    _fd_check(oracle_mod, prog_g, prog_l, ins, param_idx=[2, 3, 4, 5, 6, 7], grad_slots=[7, 8, 9, 10, 11, 12])


def test_residual_gradients_match_finite_differences(oracle_mod):
    width, layers, batch = 4, 3, 3
    prog_g = programs.residual_step(width, layers, batch, "f32", lr=0.0, return_grads=True)
    prog_l = programs.residual_step(width, layers, batch, "f32", lr=0.0)
    ins = [a.astype(np.float64) for a in synth.residual_inputs(3, width, layers, batch, "f32")]
    # wider weights so the residual branches matter
    ins = [a * (4.0 if i >= 2 else 1.0) for i, a in enumerate(ins)]
    _preacts_away_from_kinks(oracle_mod, prog_l, ins)
    n_out = 1 + 2 * layers
    _fd_check(oracle_mod, prog_g, prog_l, ins, param_idx=list(range(2, 2 + 2 * layers)),
              grad_slots=list(range(n_out, n_out + 2 * layers)))


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                vals[k] = np.array([float(x) for x in v])
    return vals


def test_hand_derived_step(oracle_mod):
    g = _read_golden("hand_mlp_2_2_1.txt")
    prog = programs.mlp_step((2, 2, 1), 1, "f32", lr=float(g["lr"][0]), return_grads=True)
    ins = [g["x"].reshape(1, 2), g["t"].reshape(1, 1), g["W1"].reshape(2, 2), g["b1"],
           g["W2"].reshape(2, 1), g["b2"]]
    ins = [a.astype(np.float32) for a in ins]
    outs = oracle_mod.run(prog.text(), [a.copy() for a in ins])
    loss, W1n, b1n, W2n, b2n, gW1, gb1, gW2, gb2 = outs
    assert loss == g["loss"][0]
    for got, key in [(W1n, "W1_new"), (b1n, "b1_new"), (W2n, "W2_new"), (b2n, "b2_new"),
                     (gW1, "gW1"), (gb1, "gb1"), (gW2, "gW2"), (gb2, "gb2")]:
        np.testing.assert_array_equal(got.ravel(), g[key].astype(np.float32), err_msg=key)


def test_sgd_closed_forms(oracle_mod):
    # zero gradient leaves W unchanged; power-of-two lr gives exact updates
    p = Program()
    W = p.input("W", "f32", (64,))
    g = p.input("g", "f32", (64,))
    p.output(p.op("sub", [W, g], "f32", alpha=0.25), inplace_of=W)
    rng = np.random.default_rng(0)
    Wv = rng.standard_normal(64).astype(np.float32)
    (out,) = oracle_mod.run(p.text(), [Wv, np.zeros(64, np.float32)])
    np.testing.assert_array_equal(out, Wv)
    gi = rng.integers(-1000, 1000, 64).astype(np.float32)
    Wi = rng.integers(-1000, 1000, 64).astype(np.float32)
    (out,) = oracle_mod.run(p.text(), [Wi, gi])
    np.testing.assert_array_equal(out, (Wi.astype(np.float64) - gi.astype(np.float64) / 4).astype(np.float32))


def test_bf16_update_stagnation(oracle_mod):
    # lr*g below half an ulp of W leaves a bf16 W bit-unchanged
    p = Program()
    W = p.input("W", "bf16", (4,))
    g = p.input("g", "bf16", (4,))
    p.output(p.op("sub", [W, g], "bf16", alpha=1e-3), inplace_of=W)
    Wv = synth._to_storage(np.array([1.0, -2.0, 0.5, 3.0]), "bf16")
    gv = synth._to_storage(np.array([1.0, -1.0, 0.5, 1.5]), "bf16")  # lr*g <= 1.5e-3 < ulp/2
    (out,) = oracle_mod.run(p.text(), [Wv, gv])
    np.testing.assert_array_equal(out, Wv)


def test_inplace_commit_is_transactional(oracle_mod):
    # The updated W aliases the input W; the second output still reads the old W.
    p = Program()
    W = p.input("W", "f32", (2, 2))
    Wn = p.op("sub", [W, 1.0], "f32")
    keep = p.op("mul", [W, 1.0], "f32")
    p.output(Wn, inplace_of=W)
    p.output(keep)
    Wv = np.array([[1, 2], [3, 4]], np.float32)
    keep_out = np.empty((2, 2), np.float32)
    oracle_mod.run(p.text(), [Wv], outputs=[Wv, keep_out])
    np.testing.assert_array_equal(Wv, [[0, 1], [2, 3]])
    np.testing.assert_array_equal(keep_out, [[1, 2], [3, 4]])


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_probe_variant_agrees_with_base(oracle_mod, cfg):
    c = dict(programs.CONFIGS[cfg])
    if cfg == "c2":
        c.update(dims=(64, 96, 80, 16), batch=24)
    base = programs.build(c)
    probe = base.probe()
    ins = programs.inputs_for(c, 1)
    o1 = oracle_mod.run(base.text(), [a.copy() for a in ins])
    o2 = oracle_mod.run(probe.text(), [a.copy() for a in ins])
    for a, b in zip(o1, o2[:len(o1)]):
        np.testing.assert_array_equal(a, b)


def test_relu_mask_in_backward(oracle_mod):
    # g_{i-1} = threshold_backward(mm(g, W^T), h, 0) is exactly 0 where h <= 0
    c = dict(programs.CONFIGS["c1"])
    probe = programs.build(c).probe()
    ins = programs.inputs_for(c, 2)
    outs = oracle_mod.run(probe.text(), ins)
    vals = {o.buf: v for o, v in zip(probe.outputs, outs)}
    h1, g1, gm1 = vals["h1"], vals["g1"], vals["gm1"]
    assert np.all(g1[h1 <= 0] == 0)
    np.testing.assert_array_equal(g1[h1 > 0], gm1[h1 > 0])
    assert (h1 <= 0).any() and (h1 > 0).any()
