"""The full-size sampled per-node check (tests/parity.py) pinned on the CPU.

Each contraction is checked at full size through a small program whose
output diagonal is the op's output at the sampled positions.  Here the
oracle's own full-size values stand in for the GPU's: the diagonal must equal
them bit for bit (every output of a contraction depends only on its own row
and column, and the oracle accumulates each output in the same k order), and
the whole sampled check must pass on them.
"""
import numpy as np
import pytest

from persistent_whole_step_amd import programs, synth

from . import parity

CASES = {
    "mlp_bf16": dict(kind="mlp", dims=(96, 160, 72, 24), batch=40, dtype="bf16", lr=1e-2),
    "residual_f16": dict(kind="residual", width=64, layers=2, batch=24, dtype="f16", lr=1e-3),
    "mlp_f32": dict(kind="mlp", dims=(40, 48, 10), batch=16, dtype="f32", lr=1e-2),
    "gemv": dict(kind="gemv", k=224, n=224, layers=2),
    "gemv_rows_xq": dict(kind="gemv", k=160, n=160, layers=2, rows=3, xq=True),
}


def _oracle_probe(oracle_mod, cfg, seed=0):
    base = programs.build(cfg)
    probe = base.probe()
    ins = programs.inputs_for(cfg, seed)
    outs = oracle_mod.run(probe.text(), [a.copy() for a in ins])
    return base, ins, parity.probe_values(base, probe, outs)


@pytest.mark.parametrize("name", list(CASES))
def test_sampled_diagonal_equals_full_oracle(oracle_mod, name):
    base, ins, vals = _oracle_probe(oracle_mod, CASES[name])
    allv = {s.buf: a for s, a in zip(base.inputs, ins)}
    allv.update(vals)
    rng = np.random.default_rng(1)
    n_mm = 0
    for op in base.ops:
        if op.opcode not in programs.CONTRACTIONS:
            continue
        m, n = op.out.shape
        rows = np.concatenate([[0, m - 1], rng.integers(0, m, 14)])
        cols = np.concatenate([[n - 1, 0], rng.integers(0, n, 14)])
        sp, arrays = parity.sampled_contraction_program(op, allv, rows, cols)
        (small,) = oracle_mod.run(sp.text(), arrays)
        d = np.arange(len(rows))
        got = small.reshape(len(rows), len(rows))[d, d]
        full = vals[op.out.buf].reshape(m, n)[rows, cols]
        parity.assert_bitexact(got, full, op.out.dtype, f"{op.name} sampled diagonal")
        n_mm += 1
    assert n_mm > 0


@pytest.mark.parametrize("name", list(CASES))
def test_sampled_check_passes_on_oracle_values(oracle_mod, name):
    base, ins, vals = _oracle_probe(oracle_mod, CASES[name])
    assert parity.check_per_node_sampled(oracle_mod, base, ins, vals, samples=24) == len(base.ops)


def test_sampled_check_catches_a_wrong_output(oracle_mod):
    """A single wrong element in a sampled position of a contraction fails."""
    base, ins, vals = _oracle_probe(oracle_mod, CASES["mlp_bf16"])
    op = next(o for o in base.ops if o.opcode in programs.CONTRACTIONS)
    bad = dict(vals)
    v = parity.f32_of(vals[op.out.buf], op.out.dtype).copy()
    v.reshape(-1)[0] = v.reshape(-1)[0] * 1.5 + 1.0  # position (0, 0) is always sampled
    bad[op.out.buf] = synth._to_storage(v.astype(np.float64), op.out.dtype)
    with pytest.raises(AssertionError):
        parity.check_per_node_sampled(oracle_mod, base, ins, bad, samples=8)
