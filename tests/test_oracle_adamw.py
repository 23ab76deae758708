"""Pins for the oracle's square root and the AdamW update (Adam with decoupled
weight decay, the optimizer the trainkernel README's "Related work and
roadmap" section names as the next one after SGD).

* sqrt: every float32 result is checked to be the correctly rounded square
  root by exact arithmetic (the square of each neighbouring midpoint is exact
  in binary64), plus the IEEE special cases;
* AdamW: hand-derived steps whose every intermediate is exact;
* AdamW against torch.optim.AdamW (an independent implementation) over
  several steps, in binary64 and in float32;
* a whole MLP step with AdamW against torch.optim.AdamW applied to the same
  step's gradients, which pins the state/parameter wiring and the in-place
  output slots.
"""
import numpy as np
import pytest

from persistent_whole_step_amd import programs, synth
from persistent_whole_step_amd.programs import AdamW, Program


def _sqrt_program(n, dtype="f32"):
    p = Program()
    x = p.input("x", "f32", (n,))
    p.output(p.op("sqrt", [x], dtype))
    return p


def test_sqrt_correctly_rounded(oracle_mod):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x7F800000, 20000, dtype=np.int64).astype(np.uint32)  # every finite positive binade
    x = np.concatenate([bits.view(np.float32),
                        np.array([1.0, 4.0, 2.0, 0.25, 1e-45, 1.1754942e-38, 3.4028235e38], np.float32)])
    (y,) = oracle_mod.run(_sqrt_program(x.size).text(), [x])
    assert np.all(np.isfinite(y)) and np.all(y > 0)
    y64 = y.astype(np.float64)
    ulp = np.spacing(y).astype(np.float64)
    lo, hi = (y64 - ulp / 2) ** 2, (y64 + ulp / 2) ** 2  # exact: 25-bit values squared
    x64 = x.astype(np.float64)
    assert np.all(lo < x64) and np.all(x64 < hi)
    assert y[-7] == 1.0 and y[-6] == 2.0 and y[-4] == 0.5


def test_sqrt_special_values(oracle_mod):
    x = np.array([0.0, -0.0, np.inf, -1.0, -np.inf, np.nan], np.float32)
    (y,) = oracle_mod.run(_sqrt_program(x.size).text(), [x])
    assert y[0] == 0 and not np.signbit(y[0])
    assert y[1] == 0 and np.signbit(y[1])
    assert y[2] == np.inf
    assert np.isnan(y[3]) and np.isnan(y[4]) and np.isnan(y[5])


def _adamw_program(n, opt, lr, wdtype="f32"):
    p = Program()
    w = p.input("w", wdtype, (n,))
    g = p.input("g", wdtype, (n,))
    m = p.input("m", "f32", (n,))
    v = p.input("v", "f32", (n,))
    c1 = p.input("c1", "f32", (1,))
    c2 = p.input("c2", "f32", (1,))
    wn, mn, vn = programs.adamw_update(p, w, g, m, v, c1, c2, lr, opt, "w")
    p.output(wn, inplace_of=w)
    p.output(mn, inplace_of=m)
    p.output(vn, inplace_of=v)
    return p


def test_adamw_hand_derived_exact(oracle_mod):
    # beta1 = 3/4, beta2 = 1/2, lr = 1/4, weight decay 2 (decay factor 1/2),
    # eps = 0, step t = 1: c1 = 4, c2 = 2.
    #   m' = 3/4 m + 1/4 g,  v' = 1/2 v + 1/2 g^2,  w' = w/2 - (m' c1) / (4 sqrt(v' c2))
    # (m, v, g) = (0, 0, 4): m' = 1, v' = 8, m'c1 = 4, sqrt(16) = 4 -> w' = w/2 - 1/4
    # (m, v, g) = (4, 9, 4): m' = 4, v' = 12.5, m'c1 = 16, sqrt(25) = 5 -> w' = w/2 - 0.8
    # (m, v, g) = (-4, 9, -4): the step flips sign -> w' = w/2 + 0.8
    # g = 0, m = 0, v = 1: m' = 0 -> only the decay acts -> w' = w/2
    opt = AdamW(beta1=0.75, beta2=0.5, eps=0.0, weight_decay=2.0)
    c1, c2 = opt.corrections(1)
    assert (c1, c2) == (4.0, 2.0)
    p = _adamw_program(4, opt, lr=0.25)
    w = np.array([1.0, 3.0, -6.0, 10.0], np.float32)
    g = np.array([4.0, 4.0, -4.0, 0.0], np.float32)
    m = np.array([0.0, 4.0, -4.0, 0.0], np.float32)
    v = np.array([0.0, 9.0, 9.0, 1.0], np.float32)
    wn, mn, vn = oracle_mod.run(p.text(), [w, g, m, v, np.float32([c1]), np.float32([c2])])
    np.testing.assert_array_equal(mn, np.float32([1.0, 4.0, -4.0, 0.0]))
    np.testing.assert_array_equal(vn, np.float32([8.0, 12.5, 12.5, 0.5]))
    step = np.float32(0.25) * (np.float32(16.0) / np.float32(5.0))  # the one rounded quotient
    np.testing.assert_array_equal(wn, np.float32([0.5 - 0.25, 1.5 - step, -3.0 + step, 5.0]))


def test_adamw_bias_corrections():
    opt = AdamW()
    c1, c2 = opt.corrections(1)
    assert c1 == np.float32(10.0) and c2 == np.float32(1000.0)
    # large t: both corrections tend to 1
    c1, c2 = opt.corrections(100000)
    assert c1 == 1.0 and c2 == 1.0
    with pytest.raises(ValueError):
        opt.corrections(0)


def _torch_adamw_steps(w, grads, opt, lr, m0, v0, t0, dtype):
    import torch
    p = torch.nn.Parameter(torch.tensor(w, dtype=dtype))
    o = torch.optim.AdamW([p], lr=lr, betas=(opt.beta1, opt.beta2), eps=opt.eps,
                          weight_decay=opt.weight_decay, foreach=False)
    o.state[p] = {"step": torch.tensor(float(t0 - 1), dtype=torch.float32),
                  "exp_avg": torch.tensor(m0, dtype=dtype), "exp_avg_sq": torch.tensor(v0, dtype=dtype)}
    out = []
    for g in grads:
        p.grad = torch.tensor(g, dtype=dtype)
        o.step()
        st = o.state[p]
        out.append((p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()))
    return out


# Hyper-parameters whose float32 values, complements (1 - beta) and decay
# factor (1 - lr * weight_decay) are all exact, so that the program's float32
# scalars state the very same optimizer torch runs in binary64.
EXACT = [(AdamW(beta1=0.875, beta2=1 - 2.0 ** -11, eps=2.0 ** -27, weight_decay=2.0 ** -4), 2.0 ** -10),
         (AdamW(beta1=0.5, beta2=0.9375, eps=2.0 ** -20, weight_decay=0.25), 2.0 ** -6)]


def _case(n=257, steps=4, seed=2):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n) for _ in range(steps)]
    m = rng.standard_normal(n) * 1e-2
    v = (rng.standard_normal(n) * 1e-2) ** 2
    return w, grads, m, v


def _oracle_steps(oracle_mod, mode, opt, lr, w, grads, m, v, t0):
    p = _adamw_program(w.size, opt, lr)
    traj = []
    for s, g in enumerate(grads):
        if mode == "f64":
            c1, c2 = 1.0 / (1.0 - opt.beta1 ** (t0 + s)), 1.0 / (1.0 - opt.beta2 ** (t0 + s))
            w, m, v = oracle_mod.run64(p.text(), [w, g, m, v, np.array([c1]), np.array([c2])])
        else:
            c1, c2 = opt.corrections(t0 + s)
            w, m, v = oracle_mod.run(p.text(), [np.float32(w), np.float32(g), np.float32(m), np.float32(v),
                                                 np.float32([c1]), np.float32([c2])])
        traj.append((w.astype(np.float64), m.astype(np.float64), v.astype(np.float64)))
    return traj


@pytest.mark.parametrize("opt,lr", EXACT)
def test_adamw_matches_torch_optim_binary64(oracle_mod, opt, lr):
    import torch
    w, grads, m, v = _case()
    want = _torch_adamw_steps(w, grads, opt, lr, m, v, 3, torch.float64)
    got = _oracle_steps(oracle_mod, "f64", opt, lr, w, grads, m, v, 3)
    for (gw, gm, gv), (tw, tm, tv) in zip(got, want):
        np.testing.assert_allclose(gm, tm, rtol=1e-13, atol=1e-18)
        np.testing.assert_allclose(gv, tv, rtol=1e-13, atol=1e-22)
        np.testing.assert_allclose(gw, tw, rtol=1e-13, atol=1e-15)


def test_adamw_float32_close_to_torch_optim(oracle_mod):
    """Default hyper-parameters (0.9, 0.999, 1e-8, 1e-2): the float32 oracle
    stays within a few float32 roundings per step of torch in binary64."""
    import torch
    opt, lr = AdamW(), 1e-3
    w, grads, m, v = _case()
    want = _torch_adamw_steps(w, grads, opt, lr, m, v, 3, torch.float64)
    got = _oracle_steps(oracle_mod, "f32", opt, lr, w, grads, m, v, 3)
    for (gw, gm, gv), (tw, tm, tv) in zip(got, want):
        # m' and w' can cancel: bound the error by the size of the state too
        np.testing.assert_allclose(gm, tm, rtol=1e-5, atol=1e-6 * np.abs(tm).max())
        np.testing.assert_allclose(gv, tv, rtol=1e-5, atol=1e-6 * np.abs(tv).max())
        np.testing.assert_allclose(gw, tw, rtol=2e-6, atol=1e-7)


def test_mlp_adamw_step_matches_torch_optim(oracle_mod):
    """One whole step: gradients from the program itself (return_grads), the
    update checked against torch.optim.AdamW per parameter, in binary64."""
    import torch
    dims, batch = (6, 5, 3), 4
    opt, lr = EXACT[0]
    prog = programs.mlp_step(dims, batch, "f32", lr, return_grads=True, optimizer=opt)
    base = synth.mlp_inputs(4, dims, batch, "f32")
    states = synth.adamw_state(5, [a.shape for a in base[2:]])
    t = 7
    c1, c2 = 1.0 / (1.0 - opt.beta1 ** t), 1.0 / (1.0 - opt.beta2 ** t)
    ins = [a.astype(np.float64) for a in base + states] + [np.array([c1]), np.array([c2])]
    outs = oracle_mod.run64(prog.text(), ins)
    n_par = 2 * (len(dims) - 1)
    # outputs: loss, params', (m', v') per param, grads
    new_p = outs[1:1 + n_par]
    new_mv = outs[1 + n_par:1 + 3 * n_par]
    grads = outs[1 + 3 * n_par:]
    for i in range(n_par):
        ((tw, tm, tv),) = _torch_adamw_steps(ins[2 + i], [grads[i]], opt, lr, ins[2 + n_par + 2 * i],
                                             ins[2 + n_par + 2 * i + 1], t, torch.float64)
        np.testing.assert_allclose(new_p[i], tw, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(new_mv[2 * i], tm, rtol=1e-13, atol=1e-18)
        np.testing.assert_allclose(new_mv[2 * i + 1], tv, rtol=1e-13, atol=1e-22)
    # in-place slots: param' -> param, m' -> m, v' -> v
    assert prog.inplace == {1 + i: 2 + i for i in range(n_par)} | {
        1 + n_par + j: 2 + n_par + j for j in range(2 * n_par)}
    # the forward/backward is the SGD program's: same loss and gradients
    sgd = programs.mlp_step(dims, batch, "f32", lr, return_grads=True)
    souts = oracle_mod.run64(sgd.text(), [a.astype(np.float64) for a in base])
    assert souts[0] == outs[0]
    for a, b in zip(souts[1 + n_par:], grads):
        np.testing.assert_array_equal(a, b)
