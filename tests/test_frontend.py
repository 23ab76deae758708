"""The capture front end (persistent_whole_step_amd.frontend) on the CPU.

A captured step is checked against the step itself run eagerly by PyTorch on
the CPU in float32: the oracle evaluates the captured program and must agree
with the eager step to within float32 accumulation-order differences.  A
mapping mistake (a transposed operand, a wrong sign or scale, a dropped
term) changes the values far beyond that.  The update mapping and the
rejection of unsupported operations are checked directly.
"""
import numpy as np
import pytest
import torch

from persistent_whole_step_amd import frontend, programs


def readme_step(weights, x, target):
    def loss(w):
        return ((torch.relu(x @ w) - target) ** 2).mean()
    gradients, value = torch.func.grad_and_value(loss)(weights)
    return value, gradients, weights - 1e-3 * gradients


def mlp_step(params, x, target):
    def loss(p):
        h = torch.relu(torch.addmm(p["b1"], x, p["W1"]))
        y = torch.addmm(p["b2"], h, p["W2"])
        return ((y - target) ** 2).mean()
    g, v = torch.func.grad_and_value(loss)(params)
    return v, {k: params[k] - 1e-2 * g[k] for k in params}


def residual_step(params, x, target):
    def loss(p):
        h = x
        for W, b in p:
            h = h + torch.relu(torch.addmm(b, h, W))
        return ((h - target) ** 2).mean()
    g, v = torch.func.grad_and_value(loss)(params)
    return v, tuple((W - 1e-2 * gW, b - 1e-2 * gb) for (W, b), (gW, gb) in zip(params, g))


def misc_step(w, x, target):
    """A step whose gradient needs div, neg, keepdim and dim-wise sums and
    means, unsqueeze and broadcast expansions."""
    def loss(v):
        h = torch.relu(x @ v)
        h = h / (h.sum(dim=1, keepdim=True) * 0.01 + 1.0)
        return ((-h + target) ** 2).mean(dim=0).sum()
    g, val = torch.func.grad_and_value(loss)(w)
    return val, w - 0.1 * g


def adamw_step(state, x, target):
    """AdamW on a one-layer model, written in torch: the state is
    (weights, m, v) and every leaf is updated."""
    w, m, v = state
    lr, b1, b2, eps, wd, c1, c2 = 1e-2, 0.9, 0.999, 1e-8, 1e-2, 1.0 / (1 - 0.9 ** 3), 1.0 / (1 - 0.999 ** 3)
    g, val = torch.func.grad_and_value(lambda u: ((torch.relu(x @ u) - target) ** 2).mean())(w)
    m2 = m * b1 + g * (1 - b1)
    v2 = v * b2 + (g * g) * (1 - b2)
    w2 = w * (1 - lr * wd) - lr * (m2 * c1) / (torch.sqrt(v2 * c2) + eps)
    return val, (w2, m2, v2)


def _examples(name, seed=0):
    gen = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen)
    if name == "readme":
        return (r(24, 16) / 5, r(8, 24), r(8, 16))
    if name == "adamw":
        return ((r(24, 16) / 5, r(24, 16) / 100, r(24, 16).abs() / 100), r(8, 24), r(8, 16))
    if name == "misc":
        return (r(24, 16) / 5, r(8, 24), r(8, 16))
    if name == "mlp":
        return ({"W1": r(24, 40) / 5, "b1": r(40) / 5, "W2": r(40, 16) / 6, "b2": r(16) / 6}, r(12, 24), r(12, 16))
    return (tuple((r(32, 32) / 8, r(32) / 8) for _ in range(3)), r(10, 32), r(10, 32))


STEPS = {"readme": readme_step, "mlp": mlp_step, "residual": residual_step, "misc": misc_step,
         "adamw": adamw_step}


def _storage(t):
    return t.detach().numpy().astype(np.float32)


@pytest.mark.parametrize("name", list(STEPS))
def test_captured_program_matches_eager_step(oracle_mod, name):
    fn, ex = STEPS[name], _examples(name)
    prog, out_spec = frontend.capture(fn, ex)
    from torch.utils import _pytree as pytree
    leaves, _ = pytree.tree_flatten(ex)
    got = oracle_mod.run(prog.text(), [_storage(t) for t in leaves])
    want, spec = pytree.tree_flatten(fn(*ex))
    assert spec == out_spec and len(got) == len(want)
    for g, w in zip(got, want):
        w = w.detach().numpy()
        assert g.shape == w.shape
        np.testing.assert_allclose(g, w, rtol=2e-4, atol=2e-6)


def test_update_mapping_marks_the_updated_state_only():
    c = frontend._capture(readme_step, _examples("readme"))
    # outputs: value, gradients, updated weights; inputs: weights, x, target
    assert frontend._update_mapping(c) == {2: 0}
    c = frontend._capture(mlp_step, _examples("mlp"))
    m = frontend._update_mapping(c)
    assert sorted(m.values()) == [0, 1, 2, 3] and 0 not in m
    c = frontend._capture(residual_step, _examples("residual"))
    assert sorted(frontend._update_mapping(c).values()) == list(range(6))


def test_update_mapping_covers_optimizer_states():
    """An AdamW step written in torch commits the weights and both moment
    states in place."""
    c = frontend._capture(adamw_step, _examples("adamw"))
    assert frontend._update_mapping(c) == {1: 0, 2: 1, 3: 2}


def test_no_update_mapping_without_an_update():
    def grads_only(w, x):
        return torch.func.grad(lambda v: (x @ v).pow(2).mean())(w)
    c = frontend._capture(grads_only, (torch.randn(8, 4), torch.randn(3, 8)))
    assert frontend._update_mapping(c) == {}


def test_unsupported_operation_is_named():
    with pytest.raises(NotImplementedError, match="tanh"):
        frontend.capture(lambda x: torch.tanh(x), (torch.randn(4, 4),))


def test_plan_only_compile_of_a_captured_step():
    from persistent_whole_step_amd import tk
    c = frontend._capture(mlp_step, _examples("mlp"))
    c.program.inplace = frontend._update_mapping(c)
    q = tk.compile(c.program.text(), device=-1).query()
    assert q["n_stages"] >= 3 and q["direct_state_commits"] + q["staged_commits"] == 4


@pytest.mark.parametrize("view", ["permute(-1,-2)", "permute(0,1)", "permute(1,0)", "transpose(1,1)",
                                  "transpose(0,1)", "transpose(-1,-2)", "t()"])
def test_view_permutations_match_eager(oracle_mod, view):
    """Square weights make a missed or spurious transpose shape-correct, so
    each view form is compared with eager torch through the oracle: the
    identity forms (permute(0,1), transpose(1,1)) leave the operand as it
    is, the swaps transpose it."""
    def step(w, x):
        v = eval(f"w.{view}")
        return x @ v + v.sum(dim=0)

    gen = torch.Generator().manual_seed(4)
    w, x = torch.randn(16, 16, generator=gen), torch.randn(5, 16, generator=gen)
    prog, _ = frontend.capture(step, (w, x))
    (got,) = oracle_mod.run(prog.text(), [_storage(w), _storage(x)])
    np.testing.assert_allclose(got, step(w, x).numpy(), rtol=2e-5, atol=2e-5)


def test_rank3_permute_is_lowered_as_a_view(oracle_mod):
    def step(a):
        return a.permute(2, 0, 1) * 2.0

    a = torch.randn(2, 3, 4, generator=torch.Generator().manual_seed(6))
    prog, _ = frontend.capture(step, (a,))
    (got,) = oracle_mod.run(prog.text(), [_storage(a)])
    np.testing.assert_array_equal(got, step(a).numpy())
