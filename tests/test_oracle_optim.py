"""Pins of the AdamW oracle (oracle/optim.py) and their sensitivity.

The pins hold the oracle against torch.optim.AdamW (an independent
implementation of the published method, run on the CPU in float64), against
the closed form of the first step from zero moments, and against the
grad_scale identity.  Each planted mistake must break at least one pin.
"""
import inspect
import textwrap

import numpy as np
import pytest
import torch

from oracle import optim as oo

HP = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _torch_run(p0, grads, **hp):
    p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    for g in grads:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def _oracle_run(p0, grads, grad_scale=1.0, **hp):
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        p, m, v = oo.adamw_step(p, g, m, v, t, grad_scale=grad_scale, **hp)
    return p, m, v


def test_adamw_matches_torch_over_ten_steps():
    r = np.random.default_rng(5)
    p0 = r.standard_normal(1000)
    grads = [r.standard_normal(1000) * (0.1 + i) for i in range(10)]
    ref = _torch_run(p0, grads, **HP)
    got = _oracle_run(p0, grads, **HP)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_adamw_first_step_closed_form():
    r = np.random.default_rng(6)
    p0, g = r.standard_normal(64), r.standard_normal(64)
    hp = dict(HP, weight_decay=0.0)
    p, m, v = oo.adamw_step(p0, g, np.zeros(64), np.zeros(64), 1, **hp)
    # m_hat = g and v_hat = g^2 after one step from zero moments
    np.testing.assert_allclose(p, p0 - hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-13)
    np.testing.assert_allclose(m, (1 - hp["beta1"]) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - hp["beta2"]) * g * g, rtol=1e-15)


def test_adamw_decay_only():
    # a zero gradient leaves the moments at zero and only decays the weights
    p0 = np.linspace(-1, 1, 9)
    p, m, v = oo.adamw_step(p0, np.zeros(9), np.zeros(9), np.zeros(9), 3, **HP)
    np.testing.assert_allclose(p, p0 * (1 - HP["lr"] * HP["weight_decay"]), rtol=1e-15)
    assert not m.any() and not v.any()


def test_adamw_grad_scale():
    r = np.random.default_rng(7)
    p0 = r.standard_normal(50)
    grads = [r.standard_normal(50) for _ in range(3)]
    a = _oracle_run(p0, grads, grad_scale=0.25, **HP)
    b = _oracle_run(p0, [0.25 * g for g in grads], **HP)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-14)


PINS = [test_adamw_matches_torch_over_ten_steps, test_adamw_first_step_closed_form, test_adamw_decay_only,
        test_adamw_grad_scale]

MUTATIONS = [
    ("m_hat = m / (1.0 - beta1 ** t)", "m_hat = m"),
    ("v_hat = v / (1.0 - beta2 ** t)", "v_hat = v / (1.0 - beta1 ** t)"),
    ("p = p * (1.0 - lr * weight_decay)", "p = p * (1.0 - weight_decay)"),
    ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    ("(1.0 - beta2) * g * g", "(1.0 - beta2) * g"),
    ("np.asarray(g, np.float64) * grad_scale", "np.asarray(g, np.float64)"),
]


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_adamw_mutation_is_caught(old, new):
    src = textwrap.dedent(inspect.getsource(oo.adamw_step))
    assert src.count(old) == 1, old
    ns = dict(vars(oo))
    exec(compile(src.replace(old, new), "<mutated>", "exec"), ns)
    saved = oo.adamw_step
    oo.adamw_step = ns["adamw_step"]
    try:
        failed = 0
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed += 1
        assert failed > 0, f"no pin caught: {new}"
    finally:
        oo.adamw_step = saved
