"""The full-size sampled per-node check (tests/parity.py) pinned on the CPU.

Each contraction is checked at full size through a small program whose
outputs are the op's outputs at the sampled rows and columns.  Here the
oracle's own full-size values stand in for the GPU's: the small program's
outputs must equal them bit for bit (every output of a contraction depends
only on its own row and column, and the oracle accumulates each output in the
same k order), the whole sampled check must pass on them, and a wrong value
planted in any one 64x64 tile of a contraction's output (the oracle's values
with a mistake put in on the CPU) must fail it.
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
def test_sampled_block_equals_full_oracle(oracle_mod, name):
    base, ins, vals = _oracle_probe(oracle_mod, CASES[name])
    allv = {s.buf: a for s, a in zip(base.inputs, ins)}
    allv.update(vals)
    rng = np.random.default_rng(1)
    n_mm = 0
    for op in base.ops:
        if op.opcode not in programs.CONTRACTIONS:
            continue
        m, n = op.out.shape
        rows, cols = parity.tile_cover(m, rng, 32), parity.tile_cover(n, rng, 32)
        sp, arrays = parity.sampled_contraction_program(op, allv, rows, cols)
        (small,) = oracle_mod.run(sp.text(), arrays)
        got = small.reshape(len(rows), len(cols))
        full = vals[op.out.buf].reshape(m, n)[rows[:, None], cols[None, :]]
        parity.assert_bitexact(got, full, op.out.dtype, f"{op.name} sampled block")
        n_mm += 1
    assert n_mm > 0


def test_tile_cover_hits_every_block():
    rng = np.random.default_rng(3)
    for n in (1, 2, 63, 64, 65, 130, 1000, 4096):
        idx = parity.tile_cover(n, rng)
        assert idx[0] == 0 and idx[-1] == n - 1 and (np.diff(idx) > 0).all()
        assert set(range((n + 63) // 64)) <= set((idx // 64).tolist())
    assert parity.tile_cover(0, rng).size == 0


@pytest.mark.parametrize("name", list(CASES))
def test_sampled_check_passes_on_oracle_values(oracle_mod, name):
    base, ins, vals = _oracle_probe(oracle_mod, CASES[name])
    assert parity.check_per_node_sampled(oracle_mod, base, ins, vals) == len(base.ops)


def _planted(vals, op, rows, cols):
    bad = dict(vals)
    v = parity.f32_of(vals[op.out.buf], op.out.dtype).copy().reshape(op.out.shape)
    v[rows, cols] = v[rows, cols] * 1.5 + 1.0
    bad[op.out.buf] = synth._to_storage(v.astype(np.float64), op.out.dtype)
    return bad


def test_sampled_check_catches_a_wrong_tile(oracle_mod):
    """A whole 64x64 output tile gone wrong (what a tile-level fault leaves)
    fails the check, wherever the tile lies."""
    cfg = dict(kind="mlp", dims=(96, 200, 72, 24), batch=136, dtype="bf16", lr=1e-2)
    base, ins, vals = _oracle_probe(oracle_mod, cfg)
    op = next(o for o in base.ops if o.opcode in programs.CONTRACTIONS)
    m, n = op.out.shape
    for tm in range(0, m, 64):
        for tn in range(0, n, 64):
            bad = _planted(vals, op, slice(tm, tm + 64), slice(tn, tn + 64))
            with pytest.raises(AssertionError):
                parity.check_per_node_sampled(oracle_mod, base, ins, bad, seed=tm + tn)


def test_sampled_check_catches_a_wrong_edge_output(oracle_mod):
    """One wrong element at a corner of a contraction's output fails."""
    base, ins, vals = _oracle_probe(oracle_mod, CASES["mlp_bf16"])
    op = next(o for o in base.ops if o.opcode in programs.CONTRACTIONS)
    m, n = op.out.shape
    for r, c in ((0, 0), (m - 1, n - 1), (0, n - 1), (m - 1, 0)):
        with pytest.raises(AssertionError):
            parity.check_per_node_sampled(oracle_mod, base, ins, _planted(vals, op, r, c))
