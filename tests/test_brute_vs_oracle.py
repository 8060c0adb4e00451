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


# ----------------------------------------------------------------------------- expert choice
def test_expert_choice_worked_example():
    """Picks worked out by hand: each column's C largest entries, the equal
    0.5s of expert 0 going to the lower token, picks held in token order."""
    p = np.array([[.5, .2], [.1, .7], [.5, .6], [.3, .1]], np.float32)
    rt, sel = O.expert_choice(p, 2)
    np.testing.assert_array_equal(rt, [[0, 2], [1, 2]])
    np.testing.assert_array_equal(sel, [[0, -1], [-1, 0], [1, 1], [-1, -1]])
    rt, sel = O.expert_choice(p, 1)
    np.testing.assert_array_equal(rt, [[0], [1]])              # 0.5 = 0.5 -> token 0
    rt, _ = O.expert_choice(p, 3)
    np.testing.assert_array_equal(rt, [[0, 2, 3], [0, 1, 2]])
    rt, sel = O.expert_choice(p, 9)                              # C > T: every token
    np.testing.assert_array_equal(rt, [[0, 1, 2, 3]] * 2)
    np.testing.assert_array_equal(sel, [[0, 0], [1, 1], [2, 2], [3, 3]])


def test_expert_choice_is_best_subset():
    """On a dyadic grid (exact sums) every expert's picks are the C-subset of
    largest total score, and among equal totals the one whose sorted tokens
    come first: that is what 'top C with ties to the lower token' means."""
    import itertools
    rng = np.random.default_rng(5)
    for trial in range(30):
        T, E = int(rng.integers(1, 8)), int(rng.integers(1, 4))
        p = (rng.integers(0, 6, size=(T, E)) / 8).astype(np.float32)   # many ties
        C = int(rng.integers(1, T + 2))
        rt, sel = O.expert_choice(p, C)
        n = min(C, T)
        for e in range(E):
            best = max(itertools.combinations(range(T), n),
                       key=lambda s: (sum(float(p[t, e]) for t in s), [-t for t in s]))
            assert rt[e].tolist() == list(best), (trial, e)
            assert sorted(np.nonzero(sel[:, e] >= 0)[0].tolist()) == list(best)
            assert [sel[t, e] for t in best] == list(range(n))


EC_CASES = [
    dict(name='ec_gelu_f32', wl=synth.Workload('h', T=16, d=8, E=4, k=2, d_ff=8, act='gelu',
                                               score='softmax', renormalize=-1, cf=1.0,
                                               dtype='f32', seed=31)),
    dict(name='ec_swiglu_bf16_cf2', wl=synth.Workload('i', T=24, d=8, E=4, k=1, d_ff=12,
                                                      act='swiglu', score='softmax',
                                                      renormalize=-1, cf=2.0, dtype='bf16',
                                                      seed=32)),
    dict(name='ec_shared_sigmoid', wl=synth.Workload('j', T=20, d=8, E=8, k=2, d_ff=4,
                                                     act='gelu', score='sigmoid', renormalize=1,
                                                     cf=1.0, dtype='bf16', seed=33, n_shared=1,
                                                     d_ff_shared=4)),
    dict(name='ec_zero_fallback', override=3, dropped_output='zero',
         wl=synth.Workload('k', T=12, d=4, E=3, k=1, d_ff=4, act='gelu', score='softmax',
                           renormalize=-1, cf=1.0, dtype='f32', seed=34)),
    dict(name='ec_capacity_over_T', override=40,
         wl=synth.Workload('l', T=10, d=4, E=3, k=1, d_ff=4, act='gelu', score='softmax',
                           renormalize=-1, cf=1.0, dtype='f32', seed=35)),
]


@pytest.mark.parametrize('case', EC_CASES, ids=[c['name'] for c in EC_CASES])
def test_expert_choice_oracle_matches_brute_force(case):
    """Expert choice: the picks equal the brute force's repeated maximum over
    tokens, every expert holds exactly min(C, T) tokens, and y is the
    per-token sum of the picking experts' outputs weighted by probability."""
    w = case['wl']
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    sh = synth.all_expert_weights(w, shared=True) if w.n_shared else None
    ov = case.get('override', 0)
    dout = case.get('dropped_output', 'residual')
    o = O.moe_forward(w, inp, ex, sh, capacity_override=ov, dropped_output=dout,
                      routing='expert')
    x, wr, lb, sb, experts, shared = _lists(w, inp, ex, sh)
    b = brute.forward(x, wr, lb, sb, experts, shared, k=w.k, act=w.act, score=w.score,
                      renormalize=w.renormalize, C=o['capacity'], dtype=w.dtype,
                      dropped_output=dout, routing='expert')
    n = min(o['capacity'], w.T)
    np.testing.assert_array_equal(o['counts'], [n] * w.E)
    np.testing.assert_array_equal(o['counts'], b['counts'])
    np.testing.assert_array_equal(o['sel'], np.array(b['sel']))
    assert o['stats']['pad'] == w.E * (o['capacity'] - n)
    assert abs(o['l_aux'] - b['l_aux']) <= 1e-12 * abs(b['l_aux'])
    yb = np.array(b['y'])
    tol = 1e-6 if w.dtype == 'f32' else 1e-2
    assert np.abs(o['y'] - yb).max() <= tol * np.abs(yb).max()
    assert np.mean(o['y'] != yb) < 0.02


def test_expert_choice_full_capacity_is_dense_mixture():
    """With C >= T every expert takes every token, so the layer is the dense
    soft mixture y_t = sum_e p_te FFN_e(x_t) over all experts; under softmax
    the balance loss is then E * sum_i (1/E) P_i = 1."""
    w = synth.Workload('m', T=12, d=8, E=4, k=1, d_ff=8, act='gelu', score='softmax',
                       renormalize=-1, cf=1.0, dtype='f32', seed=36)
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    o = O.moe_forward(w, inp, ex, capacity_override=w.T, routing='expert')
    xa = synth.as_f32(inp['x']).astype(np.float64)
    z = xa @ inp['w_router'].astype(np.float64)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dense = np.zeros_like(xa)
    for e in range(w.E):
        _, out = O.expert_ffn(xa, {kk: synth.as_f32(v[e]).astype(np.float64)
                                   for kk, v in ex.items()}, 'gelu', 'f32')
        dense += p[:, [e]] * out
    np.testing.assert_allclose(o['y'], dense, rtol=1e-5, atol=1e-6)
    assert abs(o['l_aux'] - 1.0) < 1e-12


# ----------------------------------------------------------------------------- score priority
def test_score_priority_worked_example():
    """Batch-prioritised capacity by hand: expert 0 holds tokens 0, 1, 2 with
    scores 0.3, 0.9, 0.5 and room for 2, so token 0 drops; the kept ones are
    numbered in queue order (token 1, then token 2).  Equal scores go to the
    earlier assignment in the rank-major queue (a first choice before a second
    choice)."""
    idx = np.array([[0], [0], [0], [1]])
    g = np.array([[.3], [.9], [.5], [.2]], np.float32)
    slot, dropped, counts, rt = O.assign_capacity(idx, 2, 2, 'score', g)
    np.testing.assert_array_equal(slot[:, 0], [2, 0, 1, 0])
    np.testing.assert_array_equal(dropped[:, 0], [True, False, False, False])
    np.testing.assert_array_equal(counts, [3, 1])
    np.testing.assert_array_equal(rt, [[1, 2], [3, -1]])
    idx = np.array([[0, 1], [1, 0]])
    g = np.full((2, 2), 0.5, np.float32)
    slot, dropped, _, rt = O.assign_capacity(idx, 2, 1, 'score', g)
    np.testing.assert_array_equal(dropped, [[False, True], [False, True]])   # first choices win the ties
    np.testing.assert_array_equal(rt, [[0], [1]])


def test_score_priority_properties():
    """Kept scores dominate dropped ones within each expert, counts and kept
    numbers follow C, and with room for everything the queue is the GShard one."""
    rng = np.random.default_rng(8)
    for trial in range(20):
        T, E, k = int(rng.integers(1, 60)), int(rng.integers(1, 6)), 1
        k = int(rng.integers(1, E + 1))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        g = (rng.integers(0, 5, size=(T, k)) / 4).astype(np.float32)
        C = int(rng.integers(1, T + 1))
        slot, dropped, counts, rt = O.assign_capacity(idx, E, C, 'score', g)
        np.testing.assert_array_equal(dropped, slot >= C)
        for e in range(E):
            m = idx == e
            assert sorted(slot[m].tolist()) == list(range(int(m.sum())))
            kept, drop = g[m & ~dropped], g[m & dropped]
            assert kept.size == min(C, int(m.sum()))
            if kept.size and drop.size:
                assert kept.min() >= drop.max()
        s2, d2, _, r2 = O.assign_capacity(idx, E, T, 'score', g)
        s3, d3, _, r3 = O.assign_capacity(idx, E, T, 'rank')
        np.testing.assert_array_equal(s2, s3)
        np.testing.assert_array_equal(r2, r3)


@pytest.mark.parametrize('case', [c for c in CASES if c['name'] in ('swiglu_bf16', 'top1_raw_bias', 'shared_logrank',
                                                                     'sigmoid_selbias', 'zero_fallback')],
                         ids=lambda c: c['name'])
def test_score_priority_oracle_matches_brute_force(case):
    w = case.get('wl') or synth.WORKLOADS[case['name']]
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    sh = synth.all_expert_weights(w, shared=True) if w.n_shared else None
    ov = case.get('override', 0) or max(1, O.capacity(w.T, w.k, w.E, w.cf) // 2)   # force drops
    dout = case.get('dropped_output', 'residual')
    o = O.moe_forward(w, inp, ex, sh, priority='score', capacity_override=ov, dropped_output=dout)
    x, wr, lb, sb, experts, shared = _lists(w, inp, ex, sh)
    b = brute.forward(x, wr, lb, sb, experts, shared, k=w.k, act=w.act, score=w.score,
                      renormalize=w.renormalize, C=o['capacity'], dtype=w.dtype,
                      priority='score', dropped_output=dout)
    assert o['dropped'].any()
    np.testing.assert_array_equal(o['slot'], np.array(b['slot']))
    np.testing.assert_array_equal(o['dropped'], np.array(b['dropped']))
    yb = np.array(b['y'])
    tol = 1e-6 if w.dtype == 'f32' else 1e-2
    assert np.abs(o['y'] - yb).max() <= tol * np.abs(yb).max()
    assert np.mean(o['y'] != yb) < 0.02
