"""Pins for the CPU oracle: what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, an invariant, a special case that reduces to a
library routine, or brute force on tiny inputs.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import fp32spec
from oracle import moe as O

GOLD = os.path.join(os.path.dirname(__file__), 'golden')


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- losses
def test_laux_worked_example_092():
    g = gold('laux_worked_example.json')
    E, T = g['E'], g['tokens']
    z = np.zeros((T, E), np.float32)
    z[g['tie_tokens']:, g['certain_expert']] = 1000.0     # p = (0, 1) exactly in fp64
    idx, _, probs = O.route(z, g['k'])
    assert idx[:g['tie_tokens'], 0].tolist() == [0] * g['tie_tokens']   # tie -> lower index
    l = O.load_balancing_loss(probs, idx, E)
    assert abs(l - g['expected_l_aux']) < 1e-12
    # the opposite tie rule would give the other printed value
    alt = idx.copy()
    alt[:g['tie_tokens'], 0] = 1
    assert abs(O.load_balancing_loss(probs, alt, E) - g['expected_if_ties_went_to_the_higher_index']) < 1e-12


@pytest.mark.parametrize('E,k', [(4, 1), (8, 2), (16, 4), (64, 6), (128, 8)])
def test_balanced_routing_gives_exactly_one(E, k):
    T = E * 16
    probs = np.full((T, E), 1.0 / E)               # uniform logits -> p = 1/E exactly
    np.testing.assert_array_equal(O.probabilities(np.zeros((T, E), np.float32)), probs)
    idx = np.array([[(t * k + j) % E for j in range(k)] for t in range(T)], np.int32)
    assert O.load_balancing_loss(probs, idx, E) == 1.0


@pytest.mark.parametrize('E', [2, 4, 8, 64])
def test_total_collapse_gives_E(E):
    T = 32
    z = np.zeros((T, E), np.float32)
    z[:, 0] = 1000.0                                # certain on expert 0
    idx, _, probs = O.route(z, 1)
    assert (idx == 0).all()
    assert O.load_balancing_loss(probs, idx, E) == float(E)


def test_f_divides_by_slots_not_tokens():
    # k = 2 uniform routing: dividing f by T instead of T*k would give 2.0
    E, k, T = 4, 2, 8
    probs = np.full((T, E), 0.25)
    idx = np.array([[(2 * t) % 4, (2 * t + 1) % 4] for t in range(T)], np.int32)
    assert O.load_balancing_loss(probs, idx, E) == 1.0


def test_z_loss_hand_values():
    # all-zero logits: LSE = ln E
    for E in (2, 4, 8, 128):
        assert abs(O.router_z_loss(np.zeros((3, E), np.float32)) - math.log(E) ** 2) < 1e-12
    # [0, ln 3] -> LSE = ln 4 ; [ln 3 - ln 3 ...] hand computed 2x2 case
    z = np.array([[0.0, math.log(3.0)], [1.0, 1.0]], np.float32)
    lse0 = math.log(1.0 + math.exp(float(np.float32(math.log(3.0)))))
    lse1 = 1.0 + math.log(2.0)
    assert abs(O.router_z_loss(z) - (lse0 ** 2 + lse1 ** 2) / 2) < 1e-12


# ----------------------------------------------------------------------------- softmax / gates
def test_softmax_survives_logits_of_1000():
    z = np.array([[1000.0, 0.0, -1000.0, 999.0], [-1000.0, -1000.0, -1000.0, -1000.0],
                  [1000.0, 1000.0, 1000.0, 1000.0]], np.float32)
    for score in ('softmax', 'sigmoid'):
        idx, g, p = O.route(z, 2, score)
        assert np.isfinite(p).all() and np.isfinite(g).all()
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-15)
        np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.isfinite(O.router_z_loss(z))
    assert abs(O.logsumexp(z)[0] - (1000.0 + math.log1p(math.exp(-1.0)))) < 1e-9


def test_renormalised_gates_equal_softmax_over_selected_and_sum_to_one():
    z = synth.random_logits(256, 16, seed=7, scale=3.0)
    idx, g, p = O.route(z, 4)
    # divide the full softmax by the selected mass: the page's identity
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=4 * 2.0 ** -52)


def test_top1_renormalised_gate_is_exactly_one_and_raw_gate_is_p():
    z = synth.random_logits(64, 8, seed=3, scale=2.0)
    idx, g_ren, p = O.route(z, 1, renormalize=1)
    assert (g_ren == 1.0).all()
    idx2, g_raw, p2 = O.route(z, 1)              # default for k = 1: raw
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(g_raw[:, 0], p[np.arange(64), idx[:, 0]])
    # raw gate = max of the full softmax (top-1 of logits is argmax of p)
    np.testing.assert_array_equal(g_raw[:, 0], p.max(1))


def test_top_k_matches_argsort_of_probabilities_off_ties():
    z = synth.random_logits(512, 32, seed=11)
    idx, _, p = O.route(z, 5)
    ref = np.argsort(-p, axis=1, kind='stable')[:, :5]
    np.testing.assert_array_equal(idx, ref)


def test_ties_break_by_expert_index_and_minus_zero_equals_zero():
    z = np.zeros((3, 6), np.float32)
    z[1] = np.float32(-0.0)
    z[2, ::2] = np.float32(-0.0)                 # mix of -0 and +0
    idx, g, _ = O.route(z, 3)
    assert idx.tolist() == [[0, 1, 2]] * 3
    np.testing.assert_allclose(g, 1.0 / 3, rtol=1e-15)
    z = np.array([[1.0, 2.0, 2.0, 1.0, 2.0]], np.float32)
    assert O.route(z, 4)[0].tolist() == [[1, 2, 4, 0]]


def test_shift_invariance():
    c = np.float32(37.0)
    # logits on a 1/64 grid, so that adding 37 is exact in float32
    z = np.round(synth.random_logits(128, 8, seed=5) * 64) / 64
    z = z.astype(np.float32)
    z2 = (z + c).astype(np.float32)
    assert np.array_equal(z2 - c, z)
    a, b = O.route(z, 2), O.route(z2, 2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-12)
    np.testing.assert_allclose(O.logsumexp(z2), O.logsumexp(z) + 37.0, rtol=1e-14)


def test_sigmoid_gates_and_probs():
    z = np.array([[0.0, 1.0, -2.0, 3.0], [-1000.0, -999.0, -1000.0, -998.0]], np.float32)
    idx, g, q = O.route(z, 2, score='sigmoid', renormalize=1)
    s = 1.0 / (1.0 + np.exp(-z[0].astype(np.float64)))
    assert idx[0].tolist() == [3, 1]
    np.testing.assert_allclose(g[0], s[[3, 1]] / s[[3, 1]].sum(), rtol=1e-14)
    np.testing.assert_allclose(q[0], s / s.sum(), rtol=1e-14)
    # saturated negative logits: every float32 key is 0, so the index order decides;
    # sigmoid(z) ~ e^z there, so the normalised gates are a softmax of the selected z
    assert idx[1].tolist() == [0, 1]
    e = math.exp(1.0)
    np.testing.assert_allclose(g[1], [1 / (1 + e), e / (1 + e)], rtol=1e-14)


def test_selection_bias_changes_selection_not_gates():
    z = np.array([[1.0, 0.9, 0.0, -1.0]], np.float32)
    b = np.array([0.0, 0.2, 0.0, 0.0], np.float32)
    idx, g, _ = O.route(z, 1, select_bias=b)
    assert idx.tolist() == [[1]]
    p = O.softmax(z)[0]
    assert g[0, 0] == p[1]                          # raw k=1 gate: unbiased p of the pick


# ----------------------------------------------------------------------------- sigmoid key spec
def test_spec_constants_are_what_the_header_says():
    assert Fraction(float(fp32spec.LN2_HI)) == Fraction(45426, 65536)
    assert float(fp32spec.LN2_HI) <= math.log(2) < float(fp32spec.LN2_HI) + 2.0 ** -16
    for i, c in enumerate(fp32spec.TAYLOR):
        # float32(1/i!) is the nearest float32 to the exact rational
        exact = Fraction(1, math.factorial(i))
        cf = Fraction(float(c))
        nxt = np.nextafter(c, np.float32(2)), np.nextafter(c, np.float32(0))
        assert all(abs(cf - exact) <= abs(Fraction(float(v)) - exact) for v in nxt)


def test_exp_spec_within_1p5_ulp_of_libm():
    a = np.linspace(-87.0, 88.0, 400_001).astype(np.float32)
    e = fp32spec.exp_spec(a).astype(np.float64)
    ref = np.exp(a.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(e - ref) / ulp).max() <= 1.5
    assert fp32spec.exp_spec(np.float32(0.0)) == 1.0
    assert fp32spec.exp_spec(np.float32(100.0)) == np.inf
    assert fp32spec.exp_spec(np.float32(-100.0)) == 0.0


def test_sigmoid_spec_accuracy_monotone_saturating():
    z = np.linspace(-87.0, 87.0, 400_001).astype(np.float32)
    s = fp32spec.sigmoid_spec(z).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(s - ref) / ulp).max() <= 3.0
    assert (np.diff(s) >= 0).all()
    assert fp32spec.sigmoid_spec(np.float32(0.0)) == 0.5
    assert fp32spec.sigmoid_spec(np.float32(1000.0)) == 1.0
    assert fp32spec.sigmoid_spec(np.float32(-1000.0)) == 0.0
    assert not np.isnan(fp32spec.sigmoid_spec(np.array([-1e30, 1e30], np.float32))).any()


# ----------------------------------------------------------------------------- rounding
def test_round_bf16_against_torch_and_hand_cases():
    torch = pytest.importorskip('torch')
    g = np.random.default_rng(0)
    v = np.concatenate([g.standard_normal(100_000) * 10.0 ** g.integers(-30, 30, 100_000),
                        [0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40, -1e-42]])
    v32 = v.astype(np.float32)                    # torch rounds from float32
    ours = O.round_bf16(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # direct float64 rounding (no float32 detour)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    # synth's float32 -> bf16 bits agrees
    b = synth.bf16_bits(v32)
    np.testing.assert_array_equal(synth.f32_of_bits(b).astype(np.float64), ref)


# ----------------------------------------------------------------------------- capacity
def test_capacity_examples():
    for c in gold('capacity_examples.json')['cases']:
        assert O.capacity(c['T'], c['k'], c['E'], c['cf']) == c['C']
    c = gold('capacity_examples.json')['cases'][0]
    # every first choice on expert 0: assignments #1..#1280 kept, #1281 dropped
    T, E, k = c['T'], c['E'], c['k']
    idx = np.stack([np.zeros(T, np.int32), np.arange(T, dtype=np.int32) % (E - 1) + 1], 1)
    slot, dropped, counts, _ = O.assign_capacity(idx, E, c['C'])
    n = c['first_dropped_assignment']
    assert not dropped[:n - 1, 0].any() and dropped[n - 1:, 0].all()
    assert slot[n - 1, 0] == c['C']


def test_capacity_factor_below_one_raises():
    with pytest.raises(ValueError):
        O.capacity(64, 2, 4, 0.99)
    assert O.capacity(64, 2, 4, 0.5, override=3) == 3


def test_gshard_priority_case():
    g = gold('gshard_priority.json')
    idx = np.array(g['idx'], np.int32)
    _, dr, _, _ = O.assign_capacity(idx, g['E'], g['C'], 'rank')
    assert dr.tolist() == g['rank_major_dropped']
    _, dt, _, _ = O.assign_capacity(idx, g['E'], g['C'], 'token')
    assert dt.tolist() == g['token_major_dropped']


def test_one_slot_per_expert_at_most_E_tokens_get_output():
    E, k, T = 4, 2, 32
    idx = synth.random_indices(T, E, k, seed=2)
    slot, dropped, counts, row_token = O.assign_capacity(idx, E, 1)
    served = np.unique(row_token[row_token >= 0])
    assert served.size <= E
    assert (~dropped).sum() == np.count_nonzero(counts)


@pytest.mark.parametrize('priority', ['rank', 'token'])
def test_capacity_invariants_and_stable_sort(priority):
    T, E, k = 300, 8, 3
    idx = synth.random_indices(T, E, k, seed=9, skew=0.4)
    C = 50
    slot, dropped, counts, row_token = O.assign_capacity(idx, E, C, priority)
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    # slot = position in a stable sort by expert of the priority-ordered list
    flat = idx.T.reshape(-1) if priority == 'rank' else idx.reshape(-1)
    order = np.argsort(flat, kind='stable')
    pos = np.empty_like(order)
    starts = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))[:-1]])
    pos[order] = np.arange(flat.size) - starts[flat[order]]
    ref = pos.reshape(k, T).T if priority == 'rank' else pos.reshape(T, k)
    np.testing.assert_array_equal(slot, ref)
    for e in range(E):
        ke = min(counts[e], C)
        got = slot[(idx == e) & ~dropped]
        assert sorted(got.tolist()) == list(range(ke))
        assert (row_token[e, :ke] >= 0).all() and (row_token[e, ke:] == -1).all()
        for s in range(ke):
            t = row_token[e, s]
            j = np.nonzero(idx[t] == e)[0][0]
            assert slot[t, j] == s
    assert (dropped == (slot >= C)).all()


def test_large_capacity_means_no_drops_and_batch_coupling():
    T, E, k = 200, 8, 2
    idx = synth.random_indices(T, E, k, seed=4, skew=1.0)
    _, dropped, _, _ = O.assign_capacity(idx, E, O.capacity(T, k, E, 8.0))
    assert not dropped.any()
    # a token's fate depends on its batch-mates: move the last token to the front
    C = 30
    _, d1, _, _ = O.assign_capacity(idx, E, C)
    _, d2, _, _ = O.assign_capacity(np.roll(idx, 1, axis=0), E, C)
    assert d1[-1].tolist() != d2[0].tolist() or d1.sum() == 0


# ----------------------------------------------------------------------------- params / sparsity
def test_param_table():
    for r in gold('param_table.json')['rows']:
        if r.get('dense'):
            total = active = O.ffn_params(r['d'], r['d_ff'])
        else:
            total, active = O.moe_param_counts(r['d'], r['d_ff'], r['E'], r['k'], r['n_shared'])
        assert round(total / 1e6, 1) == r['total_M']
        assert round(active / 1e6, 1) == r['active_M']
    assert O.moe_param_counts(4096, 14336, 8, 2) == (939_556_864, 234_913_792)
    assert O.moe_param_counts(1024, 512, 64, 6, 2) == (69_271_552, 8_454_144)
    assert O.ffn_params(4096, 14336) == 117_440_512


@pytest.mark.parametrize('E', [1, 2, 8, 16])
def test_top_k_equal_E_is_sparsity_one(E):
    assert O.sparsity_ratio(64, 128, E, E) == 1.0
    assert O.sparsity_ratio(64, 128, E, E, n_shared=2, act='swiglu') == 1.0


# ----------------------------------------------------------------------------- experts and combine
def test_gelu_silu_closed_forms():
    assert O.gelu(0.0) == 0.0
    u = np.linspace(-6, 6, 1001)
    np.testing.assert_allclose(O.gelu(u) - O.gelu(-u), u, rtol=0, atol=1e-15)
    assert abs(O.gelu(1.0) - 0.8413447460685429) < 1e-15         # Phi(1) = 0.841344746...
    np.testing.assert_allclose(O.silu(u) - O.silu(-u), u, rtol=0, atol=1e-14)
    assert O.silu(0.0) == 0.0


def test_logits_closed_form_small_integers():
    # integer-valued operands: every product and sum is exact, so z is exact
    g = np.random.default_rng(1)
    x = g.integers(-8, 8, (20, 24)).astype(np.float32)
    w = g.integers(-8, 8, (24, 5)).astype(np.float32)
    b = g.integers(-3, 3, 5).astype(np.float32)
    z = O.router_logits(x, w, b)
    ref = (x.astype(np.int64) @ w.astype(np.int64) + b.astype(np.int64)).astype(np.float32)
    np.testing.assert_array_equal(z, ref)


def _tiny_layer(T, d, E, k, F, act, score='softmax', dtype='f32', n_shared=0, seed=0, cf=2.0):
    w = synth.Workload('t', T=T, d=d, E=E, k=k, d_ff=F, act=act, score=score, renormalize=-1,
                       cf=cf, dtype=dtype, seed=seed, n_shared=n_shared, d_ff_shared=F)
    return w, synth.router_inputs(w), synth.all_expert_weights(w), \
        (synth.all_expert_weights(w, shared=True) if n_shared else None)


def test_k_equals_E_no_drops_is_dense_soft_mixture():
    w, inp, ex, _ = _tiny_layer(T=40, d=16, E=4, k=4, F=24, act='gelu', cf=1.0)
    out = O.moe_forward(w, inp, ex)
    assert not out['dropped'].any()
    x = synth.as_f32(inp['x']).astype(np.float64)
    p = O.probabilities(out['logits'])
    dense = np.zeros_like(x)
    for e in range(4):
        _, o = O.expert_ffn(x, {kk: v[e] for kk, v in ex.items()}, 'gelu', 'f32')
        dense += p[:, e:e + 1] * o
    np.testing.assert_allclose(out['y'], O.round_store(dense, 'f32'), rtol=0,
                               atol=2e-6 * np.abs(dense).max())


def test_shared_experts_equal_one_concatenated_expert():
    w, inp, ex, sh = _tiny_layer(T=24, d=16, E=4, k=2, F=8, act='gelu', n_shared=2)
    x = synth.as_f32(inp['x']).astype(np.float64)
    cat = dict(w_in=np.concatenate([sh['w_in'][0], sh['w_in'][1]], 0),
               b_in=np.concatenate([sh['b_in'][0], sh['b_in'][1]]),
               w_out=np.concatenate([sh['w_out'][0], sh['w_out'][1]], 1),
               b_out=sh['b_out'][0] + sh['b_out'][1])
    sep = sum(O.expert_ffn(x, {kk: v[s] for kk, v in sh.items()}, 'gelu', 'f32')[1]
              for s in range(2))
    _, one = O.expert_ffn(x, cat, 'gelu', 'f32')
    np.testing.assert_allclose(sep, one, rtol=0, atol=1e-6 * np.abs(one).max())


def test_fully_dropped_token_passes_through_and_dropped_slot_contributes_nothing():
    w, inp, ex, _ = _tiny_layer(T=30, d=8, E=4, k=2, F=8, act='gelu', cf=1.0)
    out = O.moe_forward(w, inp, ex, capacity_override=1)
    x = synth.as_f32(inp['x']).astype(np.float64)
    fb = out['dropped'].all(1)
    assert fb.sum() >= 30 - 8
    np.testing.assert_array_equal(out['y'][fb], x[fb])
    zero = O.moe_forward(w, inp, ex, capacity_override=1, dropped_output='zero')
    assert (zero['y'][fb] == 0).all()
    # a partially dropped token keeps only its surviving gated output, unrenormalised
    part = np.nonzero(out['dropped'].any(1) & ~fb)[0]
    for t in part:
        j = int(np.nonzero(~out['dropped'][t])[0][0])
        e = out['idx'][t, j]
        _, o = O.expert_ffn(x[t:t + 1], {kk: v[e] for kk, v in ex.items()}, 'gelu', 'f32')
        np.testing.assert_allclose(out['y'][t], O.round_store(out['gates'][t, j] * o[0], 'f32'),
                                   rtol=1e-6, atol=1e-7)
    assert out['stats']['fallback'] == int(fb.sum())
    assert out['stats']['kept'] + out['stats']['dropped'] == 60
    assert out['stats']['pad'] == 4 * 1 - out['stats']['kept']


def test_sampled_rows_equal_full_rows():
    w, inp, ex, _ = _tiny_layer(T=50, d=8, E=4, k=2, F=16, act='swiglu', dtype='bf16', cf=1.25)
    full = O.moe_forward(w, inp, ex)
    rows = np.array([0, 7, 8, 31, 49])
    part = O.moe_forward(w, inp, ex, rows=rows)
    np.testing.assert_array_equal(part['y'], full['y'][rows])


# ----------------------------------------------------------------------------- balancing variants
def test_sequence_loss_worked_example():
    """Worked by hand (E = 2, k = 1, two sequences of two tokens).
    Sequence 1: both tokens to expert 0 with p = (1, 0): f = (1, 0), P = (1, 0),
    loss 2 * 1 = 2.  Sequence 2: one token to each expert, p = (1/2, 1/2):
    f = P = (1/2, 1/2), loss 2 * (1/4 + 1/4) = 1.  Mean 1.5; over the whole
    batch f = P = (3/4, 1/4) would give 2 * (9/16 + 1/16) = 1.25."""
    probs = np.array([[1, 0], [1, 0], [0.5, 0.5], [0.5, 0.5]])
    idx = np.array([[0], [0], [0], [1]])
    assert O.sequence_aux_loss(probs, idx, 2, 2) == 1.5
    assert O.sequence_aux_loss(probs, idx, 2, 4) == 1.25
    assert O.load_balancing_loss(probs, idx, 2) == 1.25
    with pytest.raises(ValueError):
        O.sequence_aux_loss(probs, idx, 2, 3)


@pytest.mark.parametrize('E,k', [(4, 1), (8, 2), (16, 4)])
def test_sequence_loss_balanced_and_collapsed(E, k):
    S, n = 2 * E, 3
    # every sequence balanced on its own (uniform probabilities): exactly 1
    idx = np.array([[(t * k + j) % E for j in range(k)] for t in range(S)] * n)
    probs = np.full((S * n, E), 1.0 / E)
    assert abs(O.sequence_aux_loss(probs, idx, E, S) - 1.0) < 1e-12
    # every sequence collapsed onto one expert with probability 1: E (each
    # sequence onto a different expert, so the batch as a whole stays balanced-ish)
    idx = np.concatenate([np.full((S, k), b % E) for b in range(n)])
    probs = np.zeros((S * n, E))
    for b in range(n):
        probs[b * S:(b + 1) * S, b % E] = 1.0
    if k == 1:
        assert abs(O.sequence_aux_loss(probs, idx, E, S) - E) < 1e-12
        assert O.load_balancing_loss(probs, idx, E) < E


def test_bias_update_hand_values():
    """Mean load T*k/E = 8*1/4 = 2: the expert with 3 choices is overloaded
    (bias - gamma), the one with 1 underloaded (+ gamma), the two at 2 keep
    theirs; each result is one float32 add."""
    b = np.array([0.1, -0.2, 0.0, 0.5], np.float32)
    got = O.update_select_bias(b, [3, 1, 2, 2], 0.001, T=8, k=1)
    want = np.array([np.float32(0.1) - np.float32(0.001), np.float32(-0.2) + np.float32(0.001),
                     np.float32(0.0), np.float32(0.5)], np.float32)
    np.testing.assert_array_equal(got, want)
    # a non-integer mean: T*k/E = 5/2, so 2 is under and 3 over
    got = O.update_select_bias(np.zeros(2, np.float32), [2, 3], 0.5, T=5, k=1)
    np.testing.assert_array_equal(got, [0.5, -0.5])
