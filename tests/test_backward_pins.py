"""Pins of the backward-pass oracle: finite differences of the forward
definition, and closed forms.

The layer is evaluated smoothly (storage type 'f64', no float32 rounding of
x, weights or logit values); wherever no choice or drop changes, the loss
L = <dy, y> + a_aux L_aux + a_z L_z is then differentiable and a central
difference of the forward pass must match the analytic gradient.
"""
import numpy as np
import pytest

import synth
from oracle import backward as B
from oracle import moe as O

ALPHA_AUX, ALPHA_Z = 0.37, 0.11


def _layer(w, seed=0):
    inp = synth.router_inputs(w)
    inp = dict(inp, x=synth.as_f32(inp['x']).astype(np.float64))
    ex = {kk: synth.as_f32(v).astype(np.float64) for kk, v in synth.all_expert_weights(w).items()}
    rng = np.random.default_rng(seed)
    # non-zero biases so their gradients are exercised
    for kk in ('b_in', 'b_out'):
        if kk in ex:
            ex[kk] = 0.1 * rng.standard_normal(ex[kk].shape)
    sh = None
    if w.n_shared:
        sh = {kk: synth.as_f32(v).astype(np.float64) for kk, v in synth.all_expert_weights(w, shared=True).items()}
        for kk in ('b_in', 'b_out'):
            sh[kk] = 0.1 * rng.standard_normal(sh[kk].shape)
    if inp.get('logit_bias') is not None:
        inp['logit_bias'] = np.asarray(inp['logit_bias'], np.float64)
    dy = rng.standard_normal((w.T, w.d))
    return inp, ex, sh, dy


def _loss(w, inp, ex, sh, dy, over):
    f = O.moe_forward(w, inp, ex, sh, exact=True, **over)
    return float((dy * f['y']).sum() + ALPHA_AUX * f['l_aux'] + ALPHA_Z * f['l_z']), f


FD_CASES = [
    ('gelu_renorm', synth.Workload('fa', T=24, d=8, E=4, k=2, d_ff=12, act='gelu', score='softmax',
                                   renormalize=-1, cf=1.25, dtype='f64', seed=51), {}),
    ('swiglu_renorm', synth.Workload('fb', T=20, d=8, E=4, k=2, d_ff=8, act='swiglu', score='softmax',
                                     renormalize=-1, cf=1.25, dtype='f64', seed=52), {}),
    ('top1_raw_bias_drops', synth.Workload('fc', T=24, d=8, E=4, k=1, d_ff=8, act='gelu', score='softmax',
                                           renormalize=-1, cf=1.0, dtype='f64', seed=53,
                                           logit_bias='first_two_plus2'), {}),
    ('sigmoid_renorm', synth.Workload('fd', T=16, d=8, E=6, k=3, d_ff=8, act='swiglu', score='sigmoid',
                                      renormalize=1, cf=1.0, dtype='f64', seed=54, select_bias=True), {}),
    ('sigmoid_raw', synth.Workload('fe', T=16, d=8, E=6, k=2, d_ff=8, act='gelu', score='sigmoid',
                                   renormalize=0, cf=1.0, dtype='f64', seed=55), {}),
    ('shared_forced_drops', synth.Workload('ff', T=16, d=8, E=4, k=2, d_ff=8, act='gelu', score='softmax',
                                           renormalize=-1, cf=1.0, dtype='f64', seed=56, n_shared=1,
                                           d_ff_shared=8), dict(capacity_override=3)),
    ('fallback_residual', synth.Workload('fg', T=16, d=8, E=4, k=2, d_ff=8, act='gelu', score='softmax',
                                         renormalize=-1, cf=1.0, dtype='f64', seed=57), dict(capacity_override=2)),
    ('tiny_f32_shape', synth.WORKLOADS['tiny_f32'].with_(dtype='f64'), {}),
]


@pytest.mark.parametrize('case', FD_CASES, ids=[c[0] for c in FD_CASES])
def test_backward_matches_finite_differences(case):
    name, w, over = case
    inp, ex, sh, dy = _layer(w)
    L0, f0 = _loss(w, inp, ex, sh, dy, over)
    g = B.moe_backward(w, inp, ex, sh, f0, dy, ALPHA_AUX, ALPHA_Z,
                       dropped_output=over.get('dropped_output', 'residual'), exact=True)
    rng = np.random.default_rng(7)
    h = 1e-6

    def check(kind, get_param, set_param, grad):
        p0 = get_param()
        v = rng.standard_normal(p0.shape)
        set_param(p0 + h * v)
        Lp, fp = _loss(w, inp, ex, sh, dy, over)
        set_param(p0 - h * v)
        Lm, fm = _loss(w, inp, ex, sh, dy, over)
        set_param(p0)
        for ff in (fp, fm):        # the choices and drops must not move inside +-h
            assert (ff['idx'] == f0['idx']).all() and (ff['dropped'] == f0['dropped']).all(), kind
        fd = (Lp - Lm) / (2 * h)
        an = float((np.asarray(grad) * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (kind, fd, an)

    def setter(d, key):
        def s(val):
            d[key] = val
        return s

    check('x', lambda: inp['x'].copy(), setter(inp, 'x'), g['dx'])
    check('w_router', lambda: np.asarray(inp['w_router'], np.float64).copy(), setter(inp, 'w_router'), g['dw_router'])
    if inp.get('logit_bias') is not None:
        check('logit_bias', lambda: inp['logit_bias'].copy(), setter(inp, 'logit_bias'), g['dlogit_bias'])
    for kk in ex:
        stacked = np.stack([g['experts'][e][kk] for e in range(w.E)])
        check('expert ' + kk, lambda kk=kk: ex[kk].copy(), setter(ex, kk), stacked)
    if sh is not None:
        for kk in sh:
            stacked = np.stack([g['shared'][s][kk] for s in range(w.n_shared)])
            check('shared ' + kk, lambda kk=kk: sh[kk].copy(), setter(sh, kk), stacked)
    # the forced-drop cases do drop, and one leaves tokens to the residual fallback
    if over.get('capacity_override'):
        assert f0['dropped'].any()
    if name == 'fallback_residual':
        assert (~(~f0['dropped']).any(axis=1)).any()


def test_renormalised_top1_gate_has_no_gradient():
    """A renormalised k = 1 gate is exactly 1, so dL/dz from the main loss is 0."""
    z = np.random.default_rng(1).standard_normal((10, 5))
    idx = np.argmax(z, axis=1)[:, None]
    dz = B.router_backward(z, idx, np.random.default_rng(2).standard_normal((10, 1)), 'softmax', 1)
    assert np.abs(dz).max() == 0.0


def test_raw_top1_gate_gradient_is_the_softmax_jacobian_row():
    """Raw k = 1 gate g = p_e: dg/dz_i = p_e (delta_ie - p_i)."""
    z = np.random.default_rng(3).standard_normal((6, 4))
    idx = np.argmax(z, axis=1)[:, None]
    dz = B.router_backward(z, idx, np.ones((6, 1)), 'softmax', 0)
    p = O.softmax(z)
    for t in range(6):
        e = idx[t, 0]
        want = p[t, e] * ((np.arange(4) == e) - p[t])
        np.testing.assert_allclose(dz[t], want, rtol=1e-13, atol=1e-16)


def test_balanced_routing_gives_no_balance_gradient_and_softmax_rows_sum_to_zero():
    """With f_i = 1/E for every expert the balance gradient vanishes
    (dL/dp is constant over experts, which softmax absorbs); any softmax-path
    gradient sums to 0 over the experts of a token (shift invariance)."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal((8, 4))
    idx = np.argsort(-z, axis=1)[:, :2]
    zero = np.zeros((8, 2))
    dz = B.router_backward(z, idx, zero, 'softmax', -1, np.full(4, 0.25), 1.0, 0.0)
    assert np.abs(dz).max() < 1e-15
    dg = rng.standard_normal((8, 2))
    dz = B.router_backward(z, idx, dg, 'softmax', -1, rng.random(4), 0.5, 0.0)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-14)
    # the z-loss is not shift invariant: LSE(z + c) = LSE(z) + c, so its rows sum to 2 LSE_t / T
    dz2 = B.router_backward(z, idx, dg, 'softmax', -1, rng.random(4), 0.5, 0.3)
    np.testing.assert_allclose(dz2.sum(axis=1), 0.3 * 2 * O.logsumexp(z) / 8, rtol=1e-12)


def test_z_loss_gradient_closed_form():
    """dL_z/dz_ti = 2 LSE_t p_ti / T; for zero logits LSE = ln E, p = 1/E."""
    T, E = 5, 8
    dz = B.router_backward(np.zeros((T, E)), np.zeros((T, 1), int), np.zeros((T, 1)), 'softmax', 0,
                           None, 0.0, 1.0)
    np.testing.assert_allclose(dz, 2 * np.log(E) / E / T, rtol=1e-14)


def test_activation_derivatives():
    u = np.linspace(-6, 6, 97)
    h = 1e-6
    np.testing.assert_allclose(B.gelu_grad(u), (O.gelu(u + h) - O.gelu(u - h)) / (2 * h), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(B.silu_grad(u), (O.silu(u + h) - O.silu(u - h)) / (2 * h), rtol=1e-7, atol=1e-9)
    assert B.gelu_grad(np.array([0.0]))[0] == 0.5 and B.silu_grad(np.array([0.0]))[0] == 0.5


@pytest.mark.parametrize('score,ren', [('softmax', -1), ('softmax', 0), ('sigmoid', 1), ('sigmoid', 0)])
def test_router_backward_on_some_rows_equals_those_rows_of_the_batch(score, ren):
    """The per-row terms depend only on the row, the batch size enters as 1/T:
    evaluating a subset of rows with n_tokens = T gives those rows of the
    whole-batch result."""
    rng = np.random.default_rng(11)
    T, E, k = 40, 6, 2
    z = rng.standard_normal((T, E))
    idx = np.argsort(-z, axis=1)[:, :k]
    dg = rng.standard_normal((T, k))
    f = rng.random(E)
    full = B.router_backward(z, idx, dg, score, ren, f, 0.3, 0.2)
    rows = np.array([0, 7, 8, 31, 39])
    part = B.router_backward(z[rows], idx[rows], dg[rows], score, ren, f, 0.3, 0.2, n_tokens=T)
    np.testing.assert_allclose(part, full[rows], rtol=1e-14, atol=1e-17)


EC_FD_CASES = [
    ('ec_gelu_softmax', synth.Workload('ea', T=24, d=8, E=4, k=2, d_ff=12, act='gelu', score='softmax',
                                       renormalize=-1, cf=1.0, dtype='f64', seed=91), {}),
    ('ec_swiglu_sigmoid', synth.Workload('eb', T=20, d=8, E=5, k=2, d_ff=8, act='swiglu', score='sigmoid',
                                         renormalize=1, cf=1.0, dtype='f64', seed=92), {}),
    ('ec_shared', synth.Workload('ec', T=16, d=8, E=4, k=1, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                                 cf=1.0, dtype='f64', seed=93, n_shared=1, d_ff_shared=8), {}),
    ('ec_fallback', synth.Workload('ed', T=16, d=8, E=4, k=1, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                                   cf=1.0, dtype='f64', seed=94), dict(capacity_override=2)),
]


@pytest.mark.parametrize('case', EC_FD_CASES, ids=[c[0] for c in EC_FD_CASES])
def test_expert_choice_backward_matches_finite_differences(case):
    """Expert choice: the gate of a pick is the router probability itself; a
    central difference of the forward definition (picks held fixed inside
    +-h) matches the analytic gradient of every parameter."""
    name, w, over = case
    over = dict(over, routing='expert')
    inp, ex, sh, dy = _layer(w)
    L0, f0 = _loss(w, inp, ex, sh, dy, over)
    g = B.moe_backward_expert_choice(w, inp, ex, sh, f0, dy, ALPHA_AUX, ALPHA_Z, exact=True)
    rng = np.random.default_rng(17)
    h = 1e-6

    def check(kind, get_param, set_param, grad):
        p0 = get_param()
        v = rng.standard_normal(p0.shape)
        set_param(p0 + h * v)
        Lp, fp = _loss(w, inp, ex, sh, dy, over)
        set_param(p0 - h * v)
        Lm, fm = _loss(w, inp, ex, sh, dy, over)
        set_param(p0)
        for ff in (fp, fm):
            assert (ff['sel'] == f0['sel']).all(), kind
        fd = (Lp - Lm) / (2 * h)
        an = float((np.asarray(grad) * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (kind, fd, an)

    def setter(d_, key):
        def s_(val):
            d_[key] = val
        return s_

    check('x', lambda: inp['x'].copy(), setter(inp, 'x'), g['dx'])
    check('w_router', lambda: np.asarray(inp['w_router'], np.float64).copy(), setter(inp, 'w_router'), g['dw_router'])
    for kk in ex:
        check('expert ' + kk, lambda kk=kk: ex[kk].copy(), setter(ex, kk), np.stack([g['experts'][e][kk]
                                                                                      for e in range(w.E)]))
    if sh is not None:
        for kk in sh:
            check('shared ' + kk, lambda kk=kk: sh[kk].copy(), setter(sh, kk),
                  np.stack([g['shared'][s_][kk] for s_ in range(w.n_shared)]))
    if name == 'ec_fallback':
        assert (~(f0['sel'] >= 0).any(axis=1)).any()                     # some token is picked by no expert
