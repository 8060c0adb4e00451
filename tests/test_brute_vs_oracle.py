"""The vectorised oracle against the independent per-token brute force.

"Equals the per-token sum of gated expert outputs" is how the Lab 18 page
("What to implement" 5) pins the layer; the brute force is that per-token
reference, run on tiny inputs.
"""
import numpy as np
import pytest

import synth
from oracle import brute
from oracle import moe as O


def _lists(w, inp, ex, sh):
    x = synth.as_f32(inp['x']).astype(np.float64).tolist()
    wr = inp['w_router'].astype(np.float64).tolist()
    lb = None if inp['logit_bias'] is None else inp['logit_bias'].astype(np.float64).tolist()
    sb = None if inp['select_bias'] is None else inp['select_bias'].astype(np.float64).tolist()

    def conv(d):
        return {kk: synth.as_f32(v).astype(np.float64).tolist() for kk, v in d.items()}
    experts = [conv({kk: v[e] for kk, v in ex.items()}) for e in range(w.E)]
    shared = [conv({kk: v[s] for kk, v in sh.items()}) for s in range(w.n_shared)] if sh else []
    return x, wr, lb, sb, experts, shared


CASES = [
    dict(name='tiny_f32'),
    dict(name='swiglu_bf16', wl=synth.Workload('a', T=24, d=8, E=4, k=2, d_ff=12, act='swiglu',
                                               score='softmax', renormalize=-1, cf=1.0,
                                               dtype='bf16', seed=21)),
    dict(name='top1_raw_bias', wl=synth.Workload('b', T=40, d=8, E=6, k=1, d_ff=8, act='gelu',
                                                 score='softmax', renormalize=-1, cf=1.0,
                                                 dtype='bf16', seed=22,
                                                 logit_bias='first_two_plus2')),
    dict(name='shared_logrank', wl=synth.Workload('c', T=20, d=8, E=8, k=3, d_ff=4, act='gelu',
                                                  score='softmax', renormalize=-1, cf=1.25,
                                                  dtype='bf16', seed=23, n_shared=2,
                                                  d_ff_shared=4, logit_bias='log_rank')),
    dict(name='sigmoid_selbias', wl=synth.Workload('d', T=30, d=8, E=8, k=3, d_ff=6,
                                                   act='swiglu', score='sigmoid', renormalize=1,
                                                   cf=1.0, dtype='bf16', seed=24,
                                                   select_bias=True)),
    dict(name='token_major_override', priority='token', override=2,
         wl=synth.Workload('e', T=16, d=8, E=4, k=2, d_ff=8, act='gelu', score='softmax',
                           renormalize=-1, cf=1.0, dtype='f32', seed=25)),
    dict(name='zero_fallback', override=1, dropped_output='zero',
         wl=synth.Workload('f', T=12, d=4, E=3, k=2, d_ff=4, act='gelu', score='softmax',
                           renormalize=-1, cf=1.0, dtype='f32', seed=26)),
    dict(name='k_equals_E', wl=synth.Workload('g', T=10, d=4, E=4, k=4, d_ff=4, act='gelu',
                                              score='softmax', renormalize=-1, cf=1.0,
                                              dtype='f32', seed=27)),
]


@pytest.mark.parametrize('case', CASES, ids=[c['name'] for c in CASES])
def test_oracle_matches_brute_force(case):
    w = case.get('wl') or synth.WORKLOADS[case['name']]
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    sh = synth.all_expert_weights(w, shared=True) if w.n_shared else None
    pr = case.get('priority', 'rank')
    ov = case.get('override', 0)
    dout = case.get('dropped_output', 'residual')
    o = O.moe_forward(w, inp, ex, sh, priority=pr, capacity_override=ov, dropped_output=dout)
    x, wr, lb, sb, experts, shared = _lists(w, inp, ex, sh)
    b = brute.forward(x, wr, lb, sb, experts, shared, k=w.k, act=w.act, score=w.score,
                      renormalize=w.renormalize, C=o['capacity'], dtype=w.dtype,
                      priority=pr, dropped_output=dout)
    z_b = np.array(b['logits'], np.float32)
    # float64 sums in a different order round to the same float32 here
    np.testing.assert_array_equal(o['logits'], z_b)
    np.testing.assert_array_equal(o['idx'], np.array(b['idx']))
    np.testing.assert_array_equal(o['slot'], np.array(b['slot']))
    np.testing.assert_array_equal(o['dropped'], np.array(b['dropped']))
    np.testing.assert_array_equal(o['counts'], np.array(b['counts']))
    np.testing.assert_allclose(o['gates'], np.array(b['gates']), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o['probs'], np.array(b['probs']), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o['lse'], np.array(b['lse']), rtol=1e-13)
    assert abs(o['l_aux'] - b['l_aux']) <= 1e-12 * abs(b['l_aux'])
    assert abs(o['l_z'] - b['l_z']) <= 1e-12 * abs(b['l_z'])
    yb = np.array(b['y'])
    # same rounding points; the float64 summation order can move a value across a
    # rounding boundary of the storage type (one float32 ulp, or one bf16 ulp)
    tol = 1e-6 if w.dtype == 'f32' else 1e-2
    assert np.abs(o['y'] - yb).max() <= tol * np.abs(yb).max()
    mism = np.mean(o['y'] != yb)
    assert mism < 0.02


def test_tiny_f32_capacity_is_40():
    w = synth.WORKLOADS['tiny_f32']
    assert O.capacity(w.T, w.k, w.E, w.cf) == 40


def test_dropless_rows_worked_example():
    """Rows worked out by hand from the definition: expert e's choices follow
    the choices of lower experts, in queue order.  Choices (token: experts)
    0: 0 1, 1: 1 2, 2: 0 2, 3: 1 0.
    Rank-major queue: expert 0 gets t0, t2 (rank 0), t3 (rank 1) -> rows 0-2;
    expert 1 gets t1, t3 (rank 0), t0 (rank 1) -> rows 3-5; expert 2 gets t1,
    t2 (rank 1) -> rows 6-7.  Token-major: expert 0 t0, t2, t3; expert 1 t0,
    t1, t3; expert 2 t1, t2."""
    idx = np.array([[0, 1], [1, 2], [0, 2], [1, 0]])
    row, counts, row_token = O.dropless_rows(idx, 3, 'rank')
    np.testing.assert_array_equal(row, [[0, 5], [3, 6], [1, 7], [4, 2]])
    np.testing.assert_array_equal(counts, [3, 3, 2])
    np.testing.assert_array_equal(row_token, [0, 2, 3, 1, 3, 0, 1, 2])
    row, _, row_token = O.dropless_rows(idx, 3, 'token')
    np.testing.assert_array_equal(row, [[0, 3], [4, 6], [1, 7], [5, 2]])
    np.testing.assert_array_equal(row_token, [0, 2, 3, 0, 1, 3, 1, 2])


@pytest.mark.parametrize('case', [c for c in CASES if c['name'] not in ('tiny_f32',)] +
                         [dict(name='tiny_f32_token', priority='token',
                               wl=synth.WORKLOADS['tiny_f32'].with_(T=32))],
                         ids=lambda c: c['name'])
def test_dropless_oracle_matches_brute_force(case):
    """Dropless: nothing is dropped, y is the per-token sum of every chosen
    expert's gated output (the brute force with no capacity limit), and the
    packed row of each choice is the count of lower experts' choices plus its
    queue position."""
    w = case.get('wl') or synth.WORKLOADS[case['name']]
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    sh = synth.all_expert_weights(w, shared=True) if w.n_shared else None
    pr = case.get('priority', 'rank')
    o = O.moe_forward(w, inp, ex, sh, priority=pr, dropless=True)
    x, wr, lb, sb, experts, shared = _lists(w, inp, ex, sh)
    b = brute.forward(x, wr, lb, sb, experts, shared, k=w.k, act=w.act, score=w.score,
                      renormalize=w.renormalize, C=w.T * w.k, dtype=w.dtype, priority=pr)
    assert not o['dropped'].any() and not np.array(b['dropped']).any()
    assert o['stats']['dropped'] == 0 and o['stats']['pad'] == 0 and o['stats']['fallback'] == 0
    np.testing.assert_array_equal(o['counts'], np.array(b['counts']))
    first = np.concatenate([[0], np.cumsum(b['counts'])[:-1]])
    bidx = np.array(b['idx'])
    np.testing.assert_array_equal(o['slot'], first[bidx] + np.array(b['slot']))
    assert sorted(o['row_token'].tolist()) == sorted(np.repeat(np.arange(w.T), w.k).tolist())
    yb = np.array(b['y'])
    tol = 1e-6 if w.dtype == 'f32' else 1e-2
    assert np.abs(o['y'] - yb).max() <= tol * np.abs(yb).max()
    assert np.mean(o['y'] != yb) < 0.02
