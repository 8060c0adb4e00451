"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Every comparison uses the same seeded inputs on both sides.  See
tests/gpu_helpers.py for the comparison rules.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe as O

from gpu_helpers import DEV, device_layer, f64_of, forward, logit_error_bound, maxrel, near_tie_tokens, np_of, record

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def moe():
    assert torch.cuda.is_available(), 'GPU tests need a GPU'
    import mixture_experts_layer_20_amd as m
    return m


def say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------------- router
ROUTE_CASES = [
    # (T, E, k, score, renorm, select_bias, scale)
    (64, 4, 2, 'softmax', -1, False, 1.0),
    (1000, 8, 2, 'softmax', -1, False, 2.0),
    (777, 16, 1, 'softmax', -1, False, 1.0),
    (777, 16, 1, 'softmax', 1, False, 1.0),
    (4096, 64, 6, 'softmax', -1, True, 1.0),
    (3001, 128, 8, 'sigmoid', 1, True, 3.0),
    (513, 128, 8, 'sigmoid', 0, False, 1.0),
    (300, 256, 32, 'softmax', -1, False, 1.0),
    (300, 256, 32, 'sigmoid', 1, True, 10.0),
    (33, 6, 6, 'softmax', -1, False, 1.0),
]


def special_rows(z):
    """Ties, signed zeros and huge logits planted in the first rows."""
    T, E = z.shape
    if T >= 8:
        z[0] = 0.0
        z[1] = np.float32(-0.0)
        z[2, ::2] = np.float32(-0.0)
        z[2, 1::2] = 0.0
        z[3] = np.float32(1000.0) * np.sign(z[3])
        z[4] = -1000.0
        z[5, :] = z[5, 0]
        z[6] = np.round(z[6])               # many exact ties
        z[7, E // 2:] = 1000.0
    return z


@pytest.mark.parametrize('case', ROUTE_CASES, ids=[f'T{c[0]}E{c[1]}k{c[2]}{c[3]}{c[4]}' for c in ROUTE_CASES])
def test_route_from_given_logits_is_bit_exact(moe, case):
    T, E, k, score, ren, sb, scale = case
    say('route', case)
    z = special_rows(synth.random_logits(T, E, seed=T + E + k, scale=scale))
    b = None
    if sb:
        b = np.random.default_rng(E).uniform(-0.1, 0.1, E).astype(np.float32)
    cfg = moe.make_config(T, 8, E, k, 8, renormalize=ren, score=score, dtype='bf16')
    zt = torch.from_numpy(z).to(DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
    probs = torch.empty(T, E, dtype=torch.float32, device=DEV)
    lse = torch.empty(T, dtype=torch.float32, device=DEV)
    moe.moe_route(cfg, None, None, None, synth.to_torch(b, DEV), zt, probs, idx, gates, lse, None)
    torch.cuda.synchronize()
    r_idx, r_g, r_p = O.route(z, k, score, ren, b)
    np.testing.assert_array_equal(np_of(idx), r_idx)
    assert maxrel(np_of(gates), r_g) <= 1e-5
    assert maxrel(np_of(probs), r_p) <= 1e-5
    assert maxrel(np_of(lse), O.logsumexp(z)) <= 1e-5


def test_sigmoid_key_matches_the_spec_bit_for_bit(moe):
    """Keys that differ only in the last bits of fp32 sigmoid decide the order:
    expert e gets logit z_e and selection bias -sigmoid_spec(z_e), so every key
    is 0 or a rounding residue, and the top-k order depends on every bit."""
    from oracle import fp32spec
    E, k = 256, 32
    z = np.linspace(-30, 30, 4096 * E).astype(np.float32).reshape(4096, E)
    rng = np.random.default_rng(3)
    z = z[rng.permutation(4096)]
    T = z.shape[0]
    for shift in (0.0, 1e-3):
        b = (-fp32spec.sigmoid_spec(z[0]) + np.float32(shift)).astype(np.float32)
        cfg = moe.make_config(T, 8, E, k, 8, score='sigmoid', renormalize=1, dtype='bf16')
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
        moe.moe_route(cfg, None, None, None, torch.from_numpy(b).to(DEV),
                      torch.from_numpy(z).to(DEV), None, idx, gates, None, None)
        torch.cuda.synchronize()
        r_idx, _, _ = O.route(z, k, 'sigmoid', 1, b)
        np.testing.assert_array_equal(np_of(idx), r_idx)


def test_router_logits_within_float32_dot_bound(moe):
    for name in ('tiny_f32', 'switch_top1_skewed', 'mixtral_8x_top2', 'deepseekmoe_fine'):
        w = synth.WORKLOADS[name]
        inp, ex, sh, dev = device_layer(w, moe)
        say('logits', name)
        cfg = moe.config_from_workload(w)
        T, E, k = w.T, w.E, w.k
        logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
        moe.moe_route(cfg, dev['x'], dev['w_router'], dev['logit_bias'], None, logits, None, idx,
                      gates, None, moe.workspace(cfg, DEV))
        torch.cuda.synchronize()
        x = synth.as_f32(inp['x'])
        zr = O.router_logits(x, inp['w_router'], inp['logit_bias'])
        bound = logit_error_bound(x, inp['w_router'], inp['logit_bias']) + \
            2.0 ** -24 * np.abs(zr.astype(np.float64))
        err = np.abs(np_of(logits).astype(np.float64) - zr.astype(np.float64))
        assert (err <= bound).all(), (err / bound).max()


# bf16 tokens with at most 16 experts take the streamed logits kernel: E not
# a multiple of 4, T not a multiple of 16 or 256, d slices that end inside a
# 32-wide k step or a 256-wide chunk, one slice of several chunks (T large
# enough for a single split), a slice count of 8 with several chunks each, and
# a logit bias
LOGIT_CASES = [
    # (T, d, E, logit_bias)
    (4097, 48, 5, ''),
    (300, 1024, 3, 'first_two_plus2'),
    (1000, 264, 16, ''),
    (70001, 1032, 6, 'log_rank'),
    (17, 8, 1, ''),
    (257, 2568, 7, 'log_rank'),
    (8192, 4096, 12, ''),
]


@pytest.mark.parametrize('case', LOGIT_CASES, ids=[f'T{c[0]}d{c[1]}E{c[2]}{c[3]}' for c in LOGIT_CASES])
def test_streamed_router_logits_within_float32_dot_bound(moe, case):
    T, d, E, lb = case
    say('streamed logits', case)
    w = synth.Workload('lg', T=T, d=d, E=E, k=1, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype='bf16', seed=T + d + E, logit_bias=lb)
    inp = synth.router_inputs(w)
    cfg = moe.config_from_workload(w)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, 1, dtype=torch.int32, device=DEV)
    gates = torch.empty(T, 1, dtype=torch.float32, device=DEV)
    moe.moe_route(cfg, synth.to_torch(inp['x'], DEV), synth.to_torch(inp['w_router'], DEV),
                  synth.to_torch(inp['logit_bias'], DEV), None, logits, None, idx, gates, None,
                  moe.workspace(cfg, DEV))
    torch.cuda.synchronize()
    x = synth.as_f32(inp['x'])
    zr = O.router_logits(x, inp['w_router'], inp['logit_bias'])
    bound = logit_error_bound(x, inp['w_router'], inp['logit_bias']) + 2.0 ** -24 * np.abs(zr.astype(np.float64))
    err = np.abs(np_of(logits).astype(np.float64) - zr.astype(np.float64))
    assert (err <= bound).all(), (err / bound).max()


# the router from bf16 tokens end to end (logits kernel, then the epilogue on
# its partial logits): its choices must be the oracle's on the logits it
# wrote, bit for bit, and its gates, probabilities and log-sum-exp within
# 1e-5; E from 1 to 16 (the streamed logits kernel) and 20 (the GEMM path),
# tokens scaled to logits near 1000 and duplicated tokens included
ROUTE_OWN_CASES = [
    # (T, d, E, k, score, renorm, select_bias)
    (1000, 264, 3, 2, 'softmax', -1, False),
    (4097, 1032, 8, 2, 'softmax', -1, True),
    (777, 520, 13, 4, 'sigmoid', 1, True),
    (2049, 2568, 16, 16, 'sigmoid', 0, False),
    (65, 64, 16, 1, 'softmax', 1, False),
    (5, 8, 1, 1, 'softmax', -1, False),
    (3000, 1024, 20, 3, 'sigmoid', 1, True),
    (600, 264, 256, 32, 'sigmoid', 1, True),      # the expert and choice limits
]


@pytest.mark.parametrize('case', ROUTE_OWN_CASES, ids=lambda c: f'T{c[0]}d{c[1]}E{c[2]}k{c[3]}{c[4]}{c[5]}')
def test_router_routes_its_own_logits_like_the_oracle(moe, case):
    T, d, E, k, score, ren, sb = case
    say('router on its own logits', case)
    w = synth.Workload('op', T=T, d=d, E=E, k=k, d_ff=8, act='gelu', score=score, renormalize=ren,
                       cf=1.0, dtype='bf16', seed=T + d + E, select_bias=sb,
                       extreme_frac=0.02, extreme_scale=400.0, dup_frac=0.05)
    inp = synth.router_inputs(w)
    cfg = moe.config_from_workload(w)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
    probs = torch.empty(T, E, dtype=torch.float32, device=DEV)
    lse = torch.empty(T, dtype=torch.float32, device=DEV)
    moe.moe_route(cfg, synth.to_torch(inp['x'], DEV), synth.to_torch(inp['w_router'], DEV), None,
                  synth.to_torch(inp['select_bias'], DEV), logits, probs, idx, gates, lse,
                  moe.workspace(cfg, DEV))
    torch.cuda.synchronize()
    z = np_of(logits)
    x = synth.as_f32(inp['x'])
    zr = O.router_logits(x, inp['w_router'])
    bound = logit_error_bound(x, inp['w_router']) + 2.0 ** -24 * np.abs(zr.astype(np.float64))
    assert (np.abs(z.astype(np.float64) - zr.astype(np.float64)) <= bound).all()
    r_idx, r_g, r_p = O.route(z, k, score, ren, inp['select_bias'])
    np.testing.assert_array_equal(np_of(idx), r_idx)
    errs = dict(gates=maxrel(np_of(gates), r_g), probs=maxrel(np_of(probs), r_p),
                lse=maxrel(np_of(lse), O.logsumexp(z)))
    for q, e in errs.items():
        record(q, e)
    assert max(errs.values()) <= 1e-5, errs


# ----------------------------------------------------------------------------- capacity / dispatch
DISPATCH_CASES = [
    # (T, E, k, C, priority, skew, d)
    (64, 4, 2, 40, 'rank', 0.0, 32),
    (1000, 8, 2, 200, 'rank', 0.5, 64),
    (1000, 8, 2, 200, 'token', 0.5, 64),
    (4097, 16, 1, 256, 'rank', 0.3, 128),
    (65, 6, 6, 1, 'rank', 0.0, 16),
    (3000, 64, 6, 300, 'rank', 0.05, 256),
    (3000, 64, 6, 300, 'token', 0.05, 256),
    (1, 4, 2, 1, 'rank', 0.0, 8),
    (2048, 256, 32, 100, 'rank', 0.01, 8),
]


@pytest.mark.parametrize('case', DISPATCH_CASES, ids=[f'T{c[0]}E{c[1]}k{c[2]}C{c[3]}{c[4]}' for c in DISPATCH_CASES])
@pytest.mark.parametrize('dtype', ['bf16', 'f32'])
def test_dispatch_bit_exact(moe, case, dtype):
    T, E, k, C, pr, skew, d = case
    say('dispatch', case, dtype)
    idx = synth.random_indices(T, E, k, seed=T * 7 + E, skew=skew)
    w = synth.Workload('d', T=T, d=d, E=E, k=k, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype=dtype, seed=T)
    x = synth.router_inputs(w)['x']
    cfg = moe.make_config(T, d, E, k, 8, capacity_override=C, priority=pr, dtype=dtype)
    xt = synth.to_torch(x, DEV)
    it = torch.from_numpy(idx).to(DEV)
    slot = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    dropped = torch.full((T, k), 9, dtype=torch.uint8, device=DEV)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((E, C), -1, dtype=torch.int32, device=DEV)
    xe = torch.zeros((E, C, d), dtype=xt.dtype, device=DEV)
    ws = moe.workspace(cfg, DEV)
    moe.moe_dispatch(cfg, xt, it, slot, dropped, counts, row_token, xe, ws)
    torch.cuda.synchronize()
    r_slot, r_drop, r_counts, r_rt = O.assign_capacity(idx, E, C, pr)
    np.testing.assert_array_equal(np_of(slot), r_slot)
    np.testing.assert_array_equal(np_of(dropped).astype(bool), r_drop)
    np.testing.assert_array_equal(np_of(counts), r_counts)
    np.testing.assert_array_equal(np_of(row_token), r_rt)
    xe_n = np_of(xe)
    for e in range(E):
        ke = min(int(r_counts[e]), C)
        np.testing.assert_array_equal(xe_n[e, :ke], x[r_rt[e, :ke]])
        assert (xe_n[e, ke:] == 0).all()        # rows past kept_e untouched


@pytest.mark.parametrize('case', [c for c in DISPATCH_CASES if c[0] > 1][:6],
                         ids=[f'T{c[0]}E{c[1]}k{c[2]}{c[4]}' for c in DISPATCH_CASES if c[0] > 1][:6])
def test_dispatch_dropless_bit_exact(moe, case):
    T, E, k, _, pr, skew, d = case
    say('dispatch dropless', case)
    idx = synth.random_indices(T, E, k, seed=T * 7 + E, skew=skew)
    w = synth.Workload('d', T=T, d=d, E=E, k=k, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype='bf16', seed=T)
    x = synth.router_inputs(w)['x']
    cfg = moe.make_config(T, d, E, k, 8, priority=pr, dtype='bf16', dropless=True)
    xt = synth.to_torch(x, DEV)
    slot = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    dropped = torch.full((T, k), 9, dtype=torch.uint8, device=DEV)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((T * k,), -1, dtype=torch.int32, device=DEV)
    xe = torch.zeros((T * k, d), dtype=xt.dtype, device=DEV)
    moe.moe_dispatch(cfg, xt, torch.from_numpy(idx).to(DEV), slot, dropped, counts, row_token, xe,
                     moe.workspace(cfg, DEV))
    torch.cuda.synchronize()
    r_row, r_counts, r_rt = O.dropless_rows(idx, E, pr)
    np.testing.assert_array_equal(np_of(slot), r_row)
    assert not np_of(dropped).any()
    np.testing.assert_array_equal(np_of(counts), r_counts)
    np.testing.assert_array_equal(np_of(row_token), r_rt)
    np.testing.assert_array_equal(np_of(xe), x[r_rt])


# ----------------------------------------------------------------------------- expert FFN
FFN_CASES = [
    # (groups, rows_per_group, rows, d, F, act, dtype)
    (5, 320, [0, 1, 37, 256, 300], 256, 384, 'gelu', 'bf16'),
    (3, 520, [520, 129, 128], 256, 256, 'swiglu', 'bf16'),
    (4, 300, [300, 257, 5, 97], 512, 384, 'gelu', 'bf16'),
    (3, 600, [600, 513, 255], 512, 256, 'swiglu', 'bf16'),
    (2, 130, [130, 64], 1024, 1408, 'swiglu', 'bf16'),
    (1, 700, None, 136, 200, 'gelu', 'bf16'),
    # K not a multiple of the 64-wide k stage: last stage 40 wide; K below one stage
    (2, 300, [300, 211], 104, 168, 'swiglu', 'bf16'),
    (3, 90, [90, 33, 0], 40, 24, 'gelu', 'bf16'),
    # more tiles than the 256 workgroups, so each runs several in turn (the
    # next tile's first stage loads while the current one finishes): ragged
    # and empty experts, partial row tiles, K of 1, 2 (ragged) and many stages
    (16, 900, [900, 899, 769, 768, 0, 300, 1, 256, 257, 900, 450, 37, 900, 128, 511, 900], 2048, 1024,
     'swiglu', 'bf16'),
    (8, 1100, [1100, 1024, 1023, 0, 700, 1, 1100, 300], 512, 4096, 'gelu', 'bf16'),
    (8, 600, [600, 512, 257, 0, 600, 3, 600, 450], 64, 4096, 'swiglu', 'bf16'),
    (8, 600, [600, 512, 257, 0, 600, 3, 600, 450], 104, 6144, 'gelu', 'bf16'),
    (4, 40, [40, 3, 0, 17], 32, 64, 'gelu', 'f32'),
    (2, 50, [50, 9], 24, 40, 'swiglu', 'f32'),
]


@pytest.mark.parametrize('case', FFN_CASES, ids=[f'G{c[0]}R{c[1]}d{c[3]}F{c[4]}{c[5]}{c[6]}' for c in FFN_CASES])
def test_expert_ffn_parity(moe, case):
    G, R, rows, d, F, act, dtype = case
    say('ffn', case)
    w = synth.Workload('f', T=G * R, d=d, E=G, k=1, d_ff=F, act=act, score='softmax', renormalize=-1,
                       cf=1.0, dtype=dtype, seed=G * 100 + d)
    a = synth.router_inputs(w)['x']                      # [G*R, d]
    ex = synth.all_expert_weights(w)
    if act == 'gelu':
        # non-zero biases so that the bias path is exercised
        g = np.random.default_rng(5)
        ex['b_in'] = (g.standard_normal(ex['b_in'].shape) * 0.1).astype(np.float32)
        ex['b_out'] = (g.standard_normal(ex['b_out'].shape) * 0.1).astype(np.float32)
        if dtype == 'bf16':
            ex['b_in'] = synth.as_f32(synth.bf16_bits(ex['b_in']))
            ex['b_out'] = synth.as_f32(synth.bf16_bits(ex['b_out']))
    cfg = moe.make_config(G * R, d, G, 1, F, act=act, dtype=dtype)
    tt = lambda v: synth.to_torch(synth.bf16_bits(v) if (dtype == 'bf16' and v.dtype == np.float32) else v, DEV)
    at = synth.to_torch(a, DEV)
    dt = at.dtype
    h = torch.full((G * R, F), 7.0, dtype=dt, device=DEV)
    out = torch.full((G * R, d), 7.0, dtype=dt, device=DEV)
    rows_t = None if rows is None else torch.tensor(rows, dtype=torch.int32, device=DEV)
    if act == 'gelu':
        moe.moe_expert_ffn(cfg, act, G, R, rows_t, at, tt(ex['w_in']), None, tt(ex['b_in']),
                           tt(ex['w_out']), tt(ex['b_out']), F, h, out)
    else:
        moe.moe_expert_ffn(cfg, act, G, R, rows_t, at, tt(ex['w_up']), tt(ex['w_gate']), None,
                           tt(ex['w_out']), None, F, h, out)
    torch.cuda.synchronize()
    hn, on = f64_of(h), f64_of(out)
    af = synth.as_f32(a).astype(np.float64)
    tol = 1e-5 if dtype == 'f32' else 2e-2

    refs = {}

    def check(hn, on, src_rows):
        for g in range(G):
            n = R if rows is None else rows[g]
            if n:
                if g not in refs:
                    wts = {kk: synth.as_f32(v[g]) for kk, v in ex.items()}
                    refs[g] = O.expert_ffn(af[src_rows(g, n)], wts, act, dtype)
                rh, ro = refs[g]
                eh, eo = maxrel(hn[g * R:g * R + n], rh), maxrel(on[g * R:g * R + n], ro)
                record('H', eh)
                record('out', eo)
                assert eh <= tol and eo <= tol, (g, eh, eo)
            assert (hn[g * R + n:(g + 1) * R] == 7.0).all() and (on[g * R + n:(g + 1) * R] == 7.0).all()
    check(hn, on, lambda g, n: slice(g * R, g * R + n))
    # the same FFN with rows gathered from a shuffled token matrix
    perm = np.random.default_rng(G + R).permutation(G * R)
    a_sh = np.ascontiguousarray(a[np.argsort(perm)])          # a_sh[perm[i]] = a[i]
    gather = perm.astype(np.int32)
    # entries at or past rows[g] are never read; give them a harmless valid row
    gather[np.arange(G * R) % R >= (np.array(rows)[np.arange(G * R) // R] if rows is not None else R)] = 0
    h.fill_(7.0)
    out.fill_(7.0)
    kw = dict(gather=torch.from_numpy(gather).to(DEV))
    if act == 'gelu':
        moe.moe_expert_ffn(cfg, act, G, R, rows_t, synth.to_torch(a_sh, DEV), tt(ex['w_in']), None,
                           tt(ex['b_in']), tt(ex['w_out']), tt(ex['b_out']), F, h, out, **kw)
    else:
        moe.moe_expert_ffn(cfg, act, G, R, rows_t, synth.to_torch(a_sh, DEV), tt(ex['w_up']),
                           tt(ex['w_gate']), None, tt(ex['w_out']), None, F, h, out, **kw)
    torch.cuda.synchronize()
    check(f64_of(h), f64_of(out), lambda g, n: slice(g * R, g * R + n))


PACKED_CASES = [
    # (rows per group, d, F, act, dtype): packed back to back, total bound T*k style
    ([0, 1, 37, 256, 300, 0, 129], 256, 384, 'gelu', 'bf16'),
    ([900, 0, 769, 3, 300, 1, 256, 257, 900, 450, 37, 128, 511, 900], 512, 1024, 'swiglu', 'bf16'),
    ([600, 512, 257, 0, 600, 3, 600, 450], 104, 2048, 'gelu', 'bf16'),
    ([40, 0, 3, 17], 32, 64, 'gelu', 'f32'),
    ([50, 9, 0], 24, 40, 'swiglu', 'f32'),
]


@pytest.mark.parametrize('case', PACKED_CASES, ids=[f'G{len(c[0])}d{c[1]}F{c[2]}{c[3]}{c[4]}' for c in PACKED_CASES])
def test_expert_ffn_packed_parity(moe, case):
    rows, d, F, act, dtype = case
    G = len(rows)
    R = sum(rows)
    total = R + 5                                       # a bound above the sum
    say('ffn packed', case)
    w = synth.Workload('p', T=max(R, 1), d=d, E=G, k=1, d_ff=F, act=act, score='softmax', renormalize=-1,
                       cf=1.0, dtype=dtype, seed=G * 100 + d + 1)
    a = synth.router_inputs(w)['x']                      # [R, d]
    ex = synth.all_expert_weights(w)
    if act == 'gelu':
        g = np.random.default_rng(6)
        ex['b_in'] = (g.standard_normal(ex['b_in'].shape) * 0.1).astype(np.float32)
        ex['b_out'] = (g.standard_normal(ex['b_out'].shape) * 0.1).astype(np.float32)
        if dtype == 'bf16':
            ex['b_in'] = synth.as_f32(synth.bf16_bits(ex['b_in']))
            ex['b_out'] = synth.as_f32(synth.bf16_bits(ex['b_out']))
    cfg = moe.make_config(max(R, 1), d, G, 1, F, act=act, dtype=dtype)
    tt = lambda v: synth.to_torch(synth.bf16_bits(v) if (dtype == 'bf16' and v.dtype == np.float32) else v, DEV)
    at = synth.to_torch(a, DEV)
    rows_t = torch.tensor(rows, dtype=torch.int32, device=DEV)
    first = np.concatenate([[0], np.cumsum(rows)[:-1]])
    af = synth.as_f32(a).astype(np.float64)
    refs = {}
    for gather in (False, True):
        h = torch.full((total, F), 7.0, dtype=at.dtype, device=DEV)
        out = torch.full((total, d), 7.0, dtype=at.dtype, device=DEV)
        kw = {}
        src = at
        order = np.arange(R)
        if gather:
            # rows gathered from a shuffled token matrix
            perm = np.random.default_rng(G + R).permutation(R)
            a_sh = np.ascontiguousarray(a[np.argsort(perm)])     # a_sh[perm[i]] = a[i]
            src = synth.to_torch(a_sh, DEV)
            kw = dict(gather=torch.from_numpy(perm.astype(np.int32)).to(DEV))
        if act == 'gelu':
            moe.moe_expert_ffn_packed(cfg, act, G, rows_t, total, src, tt(ex['w_in']), None, tt(ex['b_in']),
                                      tt(ex['w_out']), tt(ex['b_out']), F, h, out, **kw)
        else:
            moe.moe_expert_ffn_packed(cfg, act, G, rows_t, total, src, tt(ex['w_up']), tt(ex['w_gate']), None,
                                      tt(ex['w_out']), None, F, h, out, **kw)
        torch.cuda.synchronize()
        hn, on = f64_of(h), f64_of(out)
        tol = 1e-5 if dtype == 'f32' else 2e-2
        for g_ in range(G):
            n = rows[g_]
            if not n:
                continue
            if g_ not in refs:
                wts = {kk: synth.as_f32(v[g_]) for kk, v in ex.items()}
                refs[g_] = O.expert_ffn(af[first[g_]:first[g_] + n], wts, act, dtype)
            rh, ro = refs[g_]
            assert maxrel(hn[first[g_]:first[g_] + n], rh) <= tol
            assert maxrel(on[first[g_]:first[g_] + n], ro) <= tol
        # rows past the packed total are untouched
        assert (hn[R:] == 7.0).all() and (on[R:] == 7.0).all()


# ----------------------------------------------------------------------------- combine and losses
@pytest.mark.parametrize('dtype,shared,zero', [('bf16', False, 0), ('bf16', True, 0), ('f32', False, 0),
                                               ('f32', False, 1)])
def test_combine_parity(moe, dtype, shared, zero):
    T, E, k, d, C = 700, 8, 3, 256, 200
    say('combine', dtype, shared, zero)
    idx = synth.random_indices(T, E, k, seed=11, skew=0.6)
    slot, dropped, counts, rt = O.assign_capacity(idx, E, C)
    w = synth.Workload('c', T=T, d=d, E=E, k=k, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype=dtype, seed=12)
    x = synth.router_inputs(w)['x']
    w2 = w.with_(T=E * C, seed=13)
    ye = synth.router_inputs(w2)['x'].reshape(E, C, d)
    w3 = w.with_(seed=14)
    s_out = synth.router_inputs(w3)['x'] if shared else None
    g = np.random.default_rng(1).random((T, k)).astype(np.float32)
    cfg = moe.make_config(T, d, E, k, 8, capacity_override=C, dtype=dtype, dropped_output=zero,
                          n_shared=1 if shared else 0, d_ff_shared=8)
    y = torch.empty(T, d, dtype=synth.to_torch(x, DEV).dtype, device=DEV)
    moe.moe_combine(cfg, synth.to_torch(x, DEV), synth.to_torch(ye, DEV), synth.to_torch(s_out, DEV),
                    torch.from_numpy(idx).to(DEV), torch.from_numpy(g).to(DEV),
                    torch.from_numpy(slot).to(DEV), torch.from_numpy(dropped.astype(np.uint8)).to(DEV),
                    y)
    torch.cuda.synchronize()
    yef = synth.as_f32(ye).astype(np.float64)
    routed = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if not dropped[t, j]:
                routed[t] += float(g[t, j]) * yef[idx[t, j], slot[t, j]]
    xf = synth.as_f32(x).astype(np.float64)
    ref = O.combine(routed, None if s_out is None else synth.as_f32(s_out).astype(np.float64), xf,
                    (~dropped).any(1), 'zero' if zero else 'residual')
    ref = O.round_store(ref, dtype)
    yn = f64_of(y)
    record('y', maxrel(yn, ref))
    assert maxrel(yn, ref) <= (1e-5 if dtype == 'f32' else 2e-2)
    fb = ~(~dropped).any(1)
    if not shared:
        assert fb.any()
        np.testing.assert_array_equal(yn[fb], 0.0 if zero else xf[fb])


def test_combine_dropless_reads_packed_rows(moe):
    T, E, k, d = 700, 8, 3, 256
    say('combine dropless')
    idx = synth.random_indices(T, E, k, seed=17, skew=0.6)
    row, counts, _ = O.dropless_rows(idx, E, 'rank')
    w = synth.Workload('c', T=T, d=d, E=E, k=k, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype='bf16', seed=18)
    x = synth.router_inputs(w)['x']
    ye = synth.router_inputs(w.with_(T=T * k, seed=19))['x']             # [T*k, d] packed
    g = np.random.default_rng(2).random((T, k)).astype(np.float32)
    cfg = moe.make_config(T, d, E, k, 8, dtype='bf16', dropless=True)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(cfg, synth.to_torch(x, DEV), synth.to_torch(ye, DEV), None, torch.from_numpy(idx).to(DEV),
                    torch.from_numpy(g).to(DEV), torch.from_numpy(row).to(DEV),
                    torch.zeros((T, k), dtype=torch.uint8, device=DEV), y)
    torch.cuda.synchronize()
    yef = synth.as_f32(ye).astype(np.float64)
    routed = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            routed[t] += float(g[t, j]) * yef[row[t, j]]
    ref = O.round_store(O.combine(routed, None, synth.as_f32(x).astype(np.float64), np.ones(T, bool), 'residual'),
                        'bf16')
    assert maxrel(f64_of(y), ref) <= 2e-2


@pytest.mark.parametrize('T,E,k,S', [(64, 4, 2, 16), (4096, 16, 1, 512), (16384, 64, 6, 2048), (1000, 8, 2, 1000),
                                     (96, 256, 32, 32)])
def test_sequence_aux_loss_parity(moe, T, E, k, S):
    say('sequence loss', T, E, k, S)
    z = synth.random_logits(T, E, seed=T + E, scale=2.0)
    idx, _, probs = O.route(z, k)
    cfg = moe.make_config(T, 8, E, k, 8, dtype='f32')
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    moe.moe_sequence_aux_loss(cfg, S, torch.from_numpy(probs.astype(np.float32)).to(DEV),
                              torch.from_numpy(idx.astype(np.int32)).to(DEV), loss, moe.workspace(cfg, DEV))
    torch.cuda.synchronize()
    ref = O.sequence_aux_loss(probs.astype(np.float32), idx, E, S)
    assert abs(float(loss.item()) - ref) <= 1e-5 * abs(ref)
    if S == T:
        assert abs(ref - O.load_balancing_loss(probs.astype(np.float32), idx, E)) <= 1e-12 * ref


@pytest.mark.parametrize('T,E,k', [(64, 4, 2), (4096, 16, 1), (65536, 128, 8), (10, 256, 3)])
def test_select_bias_update_bit_exact(moe, T, E, k):
    say('bias update', T, E, k)
    g = np.random.default_rng(T + E)
    counts = g.integers(0, 2 * T * k // E + 2, E).astype(np.int32)
    if T * k % E == 0:
        counts[:3] = T * k // E                       # exactly at the mean: unchanged
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    cfg = moe.make_config(T, 8, E, k, 8, dtype='bf16')
    bt = torch.from_numpy(b.copy()).to(DEV)
    moe.moe_update_select_bias(cfg, torch.from_numpy(counts).to(DEV), bt, 0.001)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_of(bt), O.update_select_bias(b, counts, 0.001, T, k))


@pytest.mark.parametrize('score', ['softmax', 'sigmoid'])
def test_aux_losses_from_given_logits(moe, score):
    T, E, k = 5000, 64, 6
    z = synth.random_logits(T, E, seed=21, scale=2.0)
    z[:50] *= 500.0
    idx = synth.random_indices(T, E, k, seed=22, skew=0.1)
    cfg = moe.make_config(T, 8, E, k, 8, score=score, dtype='bf16')
    losses = torch.empty(2, dtype=torch.float32, device=DEV)
    moe.moe_aux_losses(cfg, torch.from_numpy(z).to(DEV), torch.from_numpy(idx).to(DEV), losses,
                       moe.workspace(cfg, DEV))
    torch.cuda.synchronize()
    l = np_of(losses)
    ref_aux = O.load_balancing_loss(O.probabilities(z, score), idx, E)
    ref_z = O.router_z_loss(z)
    assert abs(l[0] - ref_aux) <= 1e-5 * abs(ref_aux)
    assert abs(l[1] - ref_z) <= 1e-5 * abs(ref_z)


# ----------------------------------------------------------------------------- end to end
def _compare_forward(moe, w, rows=None, **over):
    """The whole layer against the oracle, in two runs of the oracle.

    1. The oracle's own float32 logits: the GPU's must lie within the float32
       dot-product bound of them, and every token that is not near a tie must
       choose the same experts (only near-tie tokens may route differently).
    2. The oracle run on the GPU's logits (the routing steps, capacity, experts,
       combine and losses from identical float32 logits): choices, slots, drops,
       counts and statistics bit-exact over all T; gates, probabilities and LSE
       within 1e-5 max-relative; L_aux and L_z within 1e-5 relative; y on every
       sampled row within 1e-5 (float32) or 2e-2 (bf16).
    Under score priority the kept set is decided by comparing float32 gates, so
    the slots are held bit-exact to the oracle's capacity step run on the GPU's
    own gates, and rows the oracle keeps differently only because its gates
    differ from the GPU's in the last bits are left out of the y comparison.
    """
    inp, ex, sh, dev = device_layer(w, moe)
    say('forward', w.name, over)
    cfg, out = forward(moe, w, dev, **over)
    pr = over.get('priority', 'rank')
    dout = 'zero' if over.get('dropped_output') == 'zero' else 'residual'
    cov = over.get('capacity_override', 0)
    get = (lambda e: {kk: v[e] for kk, v in ex.items()})
    gsh = None if sh is None else (lambda s: {kk: v[s] for kk, v in sh.items()})
    dl = bool(over.get('dropless', False))
    x = synth.as_f32(inp['x'])
    zg = np_of(out['logits'])

    # 1. the GPU's logits against the oracle's, and the choices they make
    zr = O.router_logits(x, inp['w_router'], inp['logit_bias'])
    bound = logit_error_bound(x, inp['w_router'], inp['logit_bias']) + 2.0 ** -24 * np.abs(zr.astype(np.float64))
    assert (np.abs(zg.astype(np.float64) - zr) <= bound).all()
    near = near_tie_tokens(zr, zg, w.k, w.score, inp['select_bias'])
    idx_own = O.route(zr, w.k, w.score, w.renormalize, inp['select_bias'])[0]
    gi = np_of(out['idx'])
    same = (gi == idx_own).all(axis=1)
    assert same[~near].all(), np.nonzero(~same & ~near)[0][:10]
    say(f'  near-tie tokens {int(near.sum())}, routed differently from the oracle\'s own logits {int((~same).sum())}')

    # 2. the oracle on the GPU's logits
    ref = O.moe_forward(w, inp, get, gsh, rows=rows, priority=pr, capacity_override=cov,
                        dropped_output=dout, dropless=dl, logits=zg)
    C = ref['capacity']
    np.testing.assert_array_equal(gi, ref['idx'])
    gs, gd, gc = np_of(out['slot']), np_of(out['dropped']).astype(bool), np_of(out['counts'])
    np.testing.assert_array_equal(gc, ref['counts'])
    rws = ref['rows']
    cmp = np.ones(rws.size, bool)
    if pr == 'score' and not dl:
        ggpu = np_of(out['gates'])
        s_g, d_g, _, _ = O.assign_capacity(gi, w.E, C, 'score', scores=ggpu)
        np.testing.assert_array_equal(gs, s_g)
        np.testing.assert_array_equal(gd, d_g)
        flip = gd != ref['dropped']
        moved = flip.any(axis=1)
        # a choice the oracle keeps differently must have its gate within the
        # float32 tolerance of its expert's C-th largest gate (the kept set
        # hinged on a last-bit difference between the two sides' gates)
        for t, j in zip(*np.nonzero(flip)):
            ge = ggpu[gi == gi[t, j]].astype(np.float64)
            kth = -np.sort(-ge)[C - 1]
            assert abs(float(ggpu[t, j]) - kth) <= 1e-5 * abs(kth), (t, j, float(ggpu[t, j]), kth)
        cmp = ~moved[rws]
        say(f'  score-priority rows kept differently through last-bit gate differences: {int(moved.sum())}')
    else:
        np.testing.assert_array_equal(gs, ref['slot'])
        np.testing.assert_array_equal(gd, ref['dropped'])
    st = np_of(out['stats']).tolist()
    want = [ref['stats'][kk] for kk in ('kept', 'dropped', 'fallback', 'pad')]
    assert st[:2] == want[:2] and st[3] == want[3]
    if pr != 'score' or dl or not moved.any():
        assert st[2] == want[2]
    l = np_of(out['losses']).astype(np.float64)
    record('L_aux', maxrel(l[0], ref['l_aux']))
    record('L_z', maxrel(l[1], ref['l_z']))
    assert abs(l[0] - ref['l_aux']) <= 1e-5 * abs(ref['l_aux'])
    assert abs(l[1] - ref['l_z']) <= 1e-5 * abs(ref['l_z'])
    say(f'  L_aux {l[0]:.7f} vs {ref["l_aux"]:.7f}, L_z {l[1]:.6f} vs {ref["l_z"]:.6f}')
    for name in ('gates', 'probs', 'lse'):
        err = maxrel(np_of(out[name]), ref[name])
        record(name, err)
        assert err <= 1e-5, (name, err)
    y = f64_of(out['y'])[rws]
    tol = 1e-5 if w.dtype == 'f32' else 2e-2
    err = maxrel(y[cmp], ref['y'][cmp])
    record('y', err)
    say(f'  y max-rel err {err:.3e} over {int(cmp.sum())} of {rws.size} rows')
    assert err <= tol
    fb = ~(~ref['dropped'][rws]).any(1) & cmp
    if w.n_shared == 0 and fb.any():
        want = 0.0 if dout == 'zero' else x[rws][fb].astype(np.float64)
        np.testing.assert_array_equal(y[fb], want)
    return cfg, out, ref


def test_forward_tiny_f32(moe):
    _compare_forward(moe, synth.WORKLOADS['tiny_f32'])


@pytest.mark.parametrize('over', [dict(), dict(priority='token'), dict(capacity_override=3),
                                  dict(capacity_override=2, dropped_output='zero')])
def test_forward_tiny_f32_variants(moe, over):
    _compare_forward(moe, synth.WORKLOADS['tiny_f32'], **over)


def test_forward_switch_top1_skewed(moe):
    cfg, out, ref = _compare_forward(moe, synth.WORKLOADS['switch_top1_skewed'])
    assert ref['stats']['fallback'] > 0.3 * 4096        # experts 0 and 1 overflow


def test_forward_deepseekmoe_fine(moe):
    _compare_forward(moe, synth.WORKLOADS['deepseekmoe_fine'], rows=np.arange(0, 16384, 7))


def test_forward_mixtral_sampled(moe):
    rows = np.sort(np.random.default_rng(0).choice(8192, 192, replace=False))
    _compare_forward(moe, synth.WORKLOADS['mixtral_8x_top2'], rows=rows)


def test_forward_sigmoid_stress_sampled(moe):
    w = synth.WORKLOADS['sigmoid_stress']
    inp = synth.router_inputs(w)
    g = np.random.default_rng(1)
    rows = np.unique(np.concatenate([g.choice(w.T, 96, replace=False), inp['extreme_rows'][:16],
                                     inp['dup_rows'][:16], inp['dup_src'][:16]]))
    _compare_forward(moe, w, rows=rows)


def test_forward_splits_the_last_round_of_the_down_projection(moe):
    # 8 experts each filled to a capacity of 9 row tiles, d = 2048 (8 column
    # tiles): the down projection has 576 tiles, a last round of 64 on 256
    # compute units, which the launch splits along k (d_ff = 4096: 2 parts of
    # 2048); compared on tokens routed to the last expert, whose tiles form
    # that round, and on others
    w = synth.Workload('tail_round', T=12000, d=2048, E=8, k=2, d_ff=4096, act='gelu', score='softmax',
                       renormalize=-1, cf=1.25, dtype='bf16', seed=41)
    inp = synth.router_inputs(w)
    z = O.router_logits(synth.as_f32(inp['x']), inp['w_router'], inp['logit_bias'])
    idx = O.route(z, w.k, w.score, w.renormalize, inp['select_bias'])[0]
    on7 = np.nonzero((idx == 7).any(axis=1))[0]
    g = np.random.default_rng(4)
    rows = np.unique(np.concatenate([g.choice(on7, 120, replace=False), g.choice(w.T, 40, replace=False)]))
    cfg, out, ref = _compare_forward(moe, w, rows=rows, capacity_override=2304)
    assert (ref['counts'] >= 2304).all()        # every expert holds 9 full row tiles


def test_forward_dropless_splits_the_last_round_of_the_down_projection(moe):
    # dropless, packed rows: 8 experts of 2,922-3,099 rows give 98 row tiles,
    # so the down projection (d = 2048: 8 column tiles) has 784 tiles and a
    # last round of 16, split along k (d_ff = 4096: 2 parts); those tiles
    # belong to the last expert, so its tokens are compared, and others
    w = synth.Workload('tail_round_dl', T=12000, d=2048, E=8, k=2, d_ff=4096, act='gelu', score='softmax',
                       renormalize=-1, cf=1.25, dtype='bf16', seed=41)
    inp = synth.router_inputs(w)
    z = O.router_logits(synth.as_f32(inp['x']), inp['w_router'], inp['logit_bias'])
    idx = O.route(z, w.k, w.score, w.renormalize, inp['select_bias'])[0]
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert sum((int(c) + 255) // 256 for c in counts) * 8 % 256 == 16     # the split round
    on7 = np.nonzero((idx == 7).any(axis=1))[0]
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([g.choice(on7, 120, replace=False), g.choice(w.T, 40, replace=False)]))
    _compare_forward(moe, w, rows=rows, dropless=True)


@pytest.mark.parametrize('T', [1, 63, 65, 0])
def test_forward_ragged_and_empty(moe, T):
    w = synth.WORKLOADS['tiny_f32'].with_(T=T, name=f'tiny_T{T}')
    if T == 0:
        inp, ex, sh, dev = device_layer(w.with_(T=1), moe)
        dev['x'] = dev['x'][:0]
        cfg, out = forward(moe, w, dev)
        assert np_of(out['counts']).tolist() == [0] * w.E
        assert np_of(out['losses']).tolist() == [0.0, 0.0]
        return
    _compare_forward(moe, w)


def test_forward_k_equals_E_bf16_swiglu(moe):
    w = synth.Workload('kE', T=300, d=128, E=4, k=4, d_ff=256, act='swiglu', score='softmax',
                       renormalize=-1, cf=1.0, dtype='bf16', seed=31)
    cfg, out, ref = _compare_forward(moe, w)
    assert not ref['dropped'].any()


LIMIT_FORWARDS = [
    # (score, renormalize, select_bias, dropless)
    ('softmax', -1, False, False),
    ('sigmoid', 1, True, True),
]


@pytest.mark.parametrize('case', LIMIT_FORWARDS, ids=lambda c: f'{c[0]}{"_dropless" if c[3] else ""}')
def test_forward_at_the_expert_and_choice_limits(moe, case):
    """E = 256 experts and k = 32 choices, the largest the configuration
    admits: the router's GEMM path over 1,024 plane rows, 32 ranks of
    capacity, 256 expert groups (the packed mode's limit when dropless) and a
    32-way combine."""
    score, renorm, sb, dl = case
    w = synth.Workload('limits', T=300, d=64, E=256, k=32, d_ff=64, act='gelu', score=score,
                       renormalize=renorm, cf=1.25, dtype='bf16', seed=41, select_bias=sb)
    cfg, out, ref = _compare_forward(moe, w, dropless=dl)
    if dl:
        assert not ref['dropped'].any()
    assert int(np_of(out['counts']).sum()) == w.T * w.k


DROPLESS_FORWARDS = [
    ('tiny_f32', dict(), None),
    ('tiny_f32', dict(priority='token'), None),
    ('switch_top1_skewed', dict(), None),
    ('deepseekmoe_fine', dict(), 'every7'),
    ('mixtral_8x_top2', dict(), 'sample'),
    ('sigmoid_stress', dict(), 'sample'),
]


@pytest.mark.parametrize('case', DROPLESS_FORWARDS, ids=[f'{c[0]}{"_" + c[1]["priority"] if c[1] else ""}'
                                                          for c in DROPLESS_FORWARDS])
def test_forward_dropless(moe, case):
    name, over, rsel = case
    w = synth.WORKLOADS[name]
    rows = None
    if rsel == 'every7':
        rows = np.arange(0, w.T, 7)
    elif rsel == 'sample':
        rows = np.sort(np.random.default_rng(3).choice(w.T, 160, replace=False))
    cfg, out, ref = _compare_forward(moe, w, rows=rows, dropless=True, **over)
    assert not ref['dropped'].any()
    assert ref['stats']['dropped'] == 0 and ref['stats']['pad'] == 0


def test_forward_events_records_the_phases_of_the_same_pass(moe):
    # moe_forward_events gives the same outputs bit for bit and records its 7
    # events in order on the stream (the phases' durations add up to the pass)
    import ctypes
    w = synth.WORKLOADS['deepseekmoe_fine'].with_(T=3000, name='events')
    inp, ex, sh, dev = device_layer(w, moe)
    _, a = forward(moe, w, dev)
    path = [ln.split()[-1] for ln in open('/proc/self/maps') if 'libamdhip64' in ln][0]
    hip = ctypes.CDLL(path)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(7):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h.value)
    cfg = moe.config_from_workload(w)
    b = moe.alloc_outputs(cfg, DEV, logits=True, probs=True, lse=True)
    moe.moe_forward(cfg, {kk: v for kk, v in dev.items() if kk != 'x'}, dev['x'], b, moe.workspace(cfg, DEV),
                    events=evs)
    torch.cuda.synchronize()
    for kk in a:
        assert torch.equal(a[kk], b[kk]), kk
    ms = []
    for i in range(6):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), evs[i], evs[i + 1]) == 0
        ms.append(f.value)
    tot = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(tot), evs[0], evs[6]) == 0
    assert all(v >= 0 for v in ms) and ms[2] > 0          # the expert FFN phase takes time
    assert abs(sum(ms) - tot.value) <= 1e-3 * max(1.0, tot.value) + 1e-3
    for h in evs:
        hip.hipEventDestroy(h)
    with pytest.raises(ValueError, match='7 event'):
        moe.moe_forward(cfg, {kk: v for kk, v in dev.items() if kk != 'x'}, dev['x'], b,
                        moe.workspace(cfg, DEV), events=evs[:3])


def test_forward_is_deterministic(moe):
    w = synth.WORKLOADS['deepseekmoe_fine'].with_(T=4000, name='det')
    inp, ex, sh, dev = device_layer(w, moe)
    _, a = forward(moe, w, dev)
    _, b = forward(moe, w, dev)
    for kk in a:
        assert torch.equal(a[kk], b[kk]), kk


# ----------------------------------------------------------------------------- expert choice
def _ec_probs(T, E, kind, seed):
    g = np.random.default_rng(seed)
    if kind == 'grid':                                   # few distinct values: ties everywhere
        return (g.integers(0, 9, size=(T, E)) / 8).astype(np.float32)
    z = g.standard_normal((T, E))
    p = np.exp(z - z.max(1, keepdims=True))
    return (p / p.sum(1, keepdims=True)).astype(np.float32)


# (T, E, C, kind): every register width of the selection kernel (T <= 8K, 16K,
# 64K) and the streamed one (T > 64K), C > T, heavy ties, E = 256
EC_SELECT_CASES = [(64, 4, 40, 'softmax'), (1000, 8, 313, 'softmax'), (8192, 8, 2560, 'softmax'),
                   (12000, 16, 1000, 'grid'), (40000, 4, 25000, 'softmax'), (70001, 2, 40000, 'softmax'),
                   (5000, 8, 1250, 'grid'), (300, 3, 1000, 'softmax'), (2048, 256, 64, 'softmax'),
                   (1, 5, 1, 'softmax')]


@pytest.mark.parametrize('case', EC_SELECT_CASES, ids=lambda c: f'T{c[0]}_E{c[1]}_C{c[2]}_{c[3]}')
def test_expert_choice_select_bit_exact(moe, case):
    T, E, C, kind = case
    say('expert choice select', case)
    p = _ec_probs(T, E, kind, seed=T + E)
    rt_ref, sel_ref = O.expert_choice(p, C)
    n = min(C, T)
    cfg = moe.make_config(T, 8, E, 1, 8, capacity_override=C, dtype='f32', routing='expert')
    ws = moe.workspace(cfg, DEV)
    rt = torch.full((E, C), -7, dtype=torch.int32, device=DEV)
    sel = torch.empty(T, E, dtype=torch.int32, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    moe.moe_expert_choice(cfg, torch.from_numpy(p).to(DEV), rt, sel, counts, ws)
    torch.cuda.synchronize()
    rtn = np_of(rt)
    np.testing.assert_array_equal(np_of(counts), [n] * E)
    np.testing.assert_array_equal(rtn[:, :n], rt_ref)
    assert (rtn[:, n:] == -7).all()                      # rows past n untouched
    np.testing.assert_array_equal(np_of(sel), sel_ref)


@pytest.mark.parametrize('E,shared,zero,dtype', [(8, False, 0, 'bf16'), (8, True, 0, 'bf16'), (130, False, 1, 'f32'),
                                                 (256, False, 0, 'f32')])
def test_combine_expert_choice_parity(moe, E, shared, zero, dtype):
    """Picks from several ballots of 64 experts, summed in expert order, and the
    fallback for tokens no expert picked."""
    T, d = 500, 128
    C = max(1, T // E)                                   # about one pick per token: some get none
    say('combine expert choice', E, shared, zero, dtype)
    p = _ec_probs(T, E, 'softmax', seed=E)
    rt, sel = O.expert_choice(p, C)
    w = synth.Workload('c', T=T, d=d, E=E, k=1, d_ff=8, act='gelu', score='softmax', renormalize=-1,
                       cf=1.0, dtype=dtype, seed=41)
    x = synth.router_inputs(w)['x']
    ye = synth.router_inputs(w.with_(T=E * C, seed=42))['x'].reshape(E, C, d)
    s_out = synth.router_inputs(w.with_(seed=43))['x'] if shared else None
    cfg = moe.make_config(T, d, E, 1, 8, capacity_override=C, dtype=dtype, dropped_output=zero,
                          n_shared=1 if shared else 0, d_ff_shared=8, routing='expert')
    y = torch.empty(T, d, dtype=synth.to_torch(x, DEV).dtype, device=DEV)
    moe.moe_combine_expert_choice(cfg, synth.to_torch(x, DEV), synth.to_torch(ye, DEV), synth.to_torch(s_out, DEV),
                                  torch.from_numpy(p).to(DEV), torch.from_numpy(sel).to(DEV), y)
    torch.cuda.synchronize()
    yef = synth.as_f32(ye).astype(np.float64)
    routed = np.zeros((T, d))
    for t in range(T):
        for e in range(E):
            if sel[t, e] >= 0:
                routed[t] += float(p[t, e]) * yef[e, sel[t, e]]
    picked = (sel >= 0).any(1)
    xf = synth.as_f32(x).astype(np.float64)
    ref = O.round_store(O.combine(routed, None if s_out is None else synth.as_f32(s_out).astype(np.float64), xf,
                                  picked, 'zero' if zero else 'residual'), dtype)
    yn = f64_of(y)
    assert maxrel(yn, ref) <= (1e-5 if dtype == 'f32' else 2e-2)
    if not shared:
        assert (~picked).any() and ((sel >= 0).sum(1) > 1).any()
        np.testing.assert_array_equal(yn[~picked], 0.0 if zero else xf[~picked])


def _compare_forward_ec(moe, w, rows=None, **over):
    """The whole layer under expert choice against the oracle.

    The GPU's logits must lie within the float32 dot-product bound of the
    oracle's own.  Given the GPU's float32 probabilities, its picks must be
    exactly the oracle's selection (n per expert, equal probabilities to the
    lower token, rows numbered in token order).  The oracle run on the GPU's
    logits gives the references at the stated bar: top-k choices bit-exact;
    gates, probabilities and LSE within 1e-5 max-relative; L_aux and L_z
    within 1e-5; statistics exact; y on the sampled rows within 1e-5 / 2e-2.
    That run forms its probabilities from the same logits with its own exp, so
    its picks may differ from the GPU's only where an expert's n-th and
    (n+1)-th probabilities differ in the last bits; such tokens are counted and
    left out of the y comparison.
    """
    inp, ex, sh, dev = device_layer(w, moe)
    say('forward expert choice', w.name, over)
    cfg, out = forward(moe, w, dev, routing='expert', **over)
    dout = 'zero' if over.get('dropped_output') == 'zero' else 'residual'
    get = (lambda e: {kk: v[e] for kk, v in ex.items()})
    gsh = None if sh is None else (lambda s: {kk: v[s] for kk, v in sh.items()})
    x = synth.as_f32(inp['x'])
    zg = np_of(out['logits'])
    zr = O.router_logits(x, inp['w_router'], inp['logit_bias'])
    bound = logit_error_bound(x, inp['w_router'], inp['logit_bias']) + 2.0 ** -24 * np.abs(zr.astype(np.float64))
    assert (np.abs(zg.astype(np.float64) - zr) <= bound).all()

    ref = O.moe_forward(w, inp, get, gsh, rows=rows, capacity_override=over.get('capacity_override', 0),
                        dropped_output=dout, routing='expert', logits=zg)
    T, E, C = w.T, w.E, ref['capacity']
    n = min(C, T)
    gp = np_of(out['probs'])
    gsel, gc = np_of(out['sel']), np_of(out['counts'])
    # the picks, bit-exact given identical float32 probabilities
    rt_g, sel_g = O.expert_choice(gp, C)
    np.testing.assert_array_equal(gsel, sel_g)
    np.testing.assert_array_equal(gc, [n] * E)
    np.testing.assert_array_equal(np_of(out['idx']), ref['idx'])
    for name in ('gates', 'probs', 'lse'):
        err = maxrel(np_of(out[name]), ref[name])
        record(name, err)
        assert err <= 1e-5, (name, err)
    # the oracle's own picks from its own probabilities of the same logits
    rp = ref['probs']
    diff = (gsel >= 0) != (ref['sel'] >= 0)
    if diff.any():
        kth = -np.sort(-rp.astype(np.float32), axis=0)[n - 1].astype(np.float64)
        band = np.abs(rp - kth[None, :]) <= 1e-5 * np.abs(kth)[None, :]
        assert band[diff].all(), np.argwhere(diff & ~band)[:5]
    tok_diff = diff.any(1)
    say(f'  tokens the oracle picks differently through last-bit probability differences: {int(tok_diff.sum())}')
    st = np_of(out['stats'])
    unpicked = int((~(gsel >= 0).any(1)).sum())
    assert st.tolist() == [E * n, 0, unpicked if w.n_shared == 0 else 0, E * (C - n)]
    if not tok_diff.any():
        assert st[2] == ref['stats']['fallback']
    l = np_of(out['losses']).astype(np.float64)
    record('L_aux', maxrel(l[0], ref['l_aux']))
    record('L_z', maxrel(l[1], ref['l_z']))
    assert abs(l[0] - ref['l_aux']) <= 1e-5 * abs(ref['l_aux'])
    assert abs(l[1] - ref['l_z']) <= 1e-5 * abs(ref['l_z'])
    rws = ref['rows']
    cmp = ~tok_diff[rws]
    y = f64_of(out['y'])[rws]
    tol = 1e-5 if w.dtype == 'f32' else 2e-2
    err = maxrel(y[cmp], ref['y'][cmp])
    record('y', err)
    say(f'  y max-rel err {err:.3e} over {int(cmp.sum())} of {rws.size} rows; L_aux {l[0]:.7f} vs {ref["l_aux"]:.7f}')
    assert err <= tol
    none = ~(ref['sel'][rws] >= 0).any(1) & cmp
    if w.n_shared == 0 and none.any():
        want = 0.0 if dout == 'zero' else x[rws][none].astype(np.float64)
        np.testing.assert_array_equal(y[none], want)
    return cfg, out, ref


EC_FORWARDS = [
    ('tiny_f32', dict(), None),
    ('tiny_f32', dict(capacity_override=5, dropped_output='zero'), None),
    ('tiny_f32', dict(capacity_override=64), None),
    ('switch_top1_skewed', dict(), 'every5'),
    ('deepseekmoe_fine', dict(), 'every7'),
    ('mixtral_8x_top2', dict(), 'sample'),
    ('sigmoid_stress', dict(), 'sample'),
]


@pytest.mark.parametrize('case', EC_FORWARDS, ids=lambda c: c[0] + ''.join(f'_{k}{v}' for k, v in c[1].items()))
def test_forward_expert_choice(moe, case):
    name, over, rsel = case
    w = synth.WORKLOADS[name]
    rows = None
    if rsel == 'every5':
        rows = np.arange(0, w.T, 5)
    elif rsel == 'every7':
        rows = np.arange(0, w.T, 7)
    elif rsel == 'sample':
        rows = np.sort(np.random.default_rng(4).choice(w.T, 128, replace=False))
    _compare_forward_ec(moe, w, rows=rows, **over)


@pytest.mark.parametrize('T', [0, 1, 65])
def test_forward_expert_choice_ragged_and_empty(moe, T):
    w = synth.WORKLOADS['tiny_f32'].with_(T=T, name=f'tiny_ec_T{T}')
    if T == 0:
        inp, ex, sh, dev = device_layer(w.with_(T=1), moe)
        dev['x'] = dev['x'][:0]
        cfg, out = forward(moe, w, dev, routing='expert')
        assert np_of(out['counts']).tolist() == [0] * w.E
        assert np_of(out['losses']).tolist() == [0.0, 0.0]
        return
    _compare_forward_ec(moe, w)



# ----------------------------------------------------------------------------- score priority
# (T, E, k, C, kind): the selection widths (lists up to 8K, 16K, 64K entries and
# the streamed path past 64K tokens), heavy gate ties, many drops
SCORE_CASES = [(700, 8, 3, 100, 'uniform'), (4096, 16, 1, 256, 'uniform'), (16384, 64, 6, 1536, 'grid'),
               (70000, 4, 2, 20000, 'uniform'), (3000, 5, 2, 400, 'grid'), (64, 4, 2, 40, 'uniform')]


@pytest.mark.parametrize('case', SCORE_CASES, ids=lambda c: f'T{c[0]}_E{c[1]}_k{c[2]}_C{c[3]}_{c[4]}')
def test_dispatch_by_score_bit_exact(moe, case):
    T, E, k, C, kind = case
    say('dispatch by score', case)
    idx = synth.random_indices(T, E, k, seed=T + k, skew=0.5)
    g = np.random.default_rng(T).random((T, k)).astype(np.float32)
    if kind == 'grid':
        g = (np.round(g * 8) / 8).astype(np.float32)
    slot_r, dropped_r, counts_r, rt_r = O.assign_capacity(idx, E, C, 'score', g)
    cfg = moe.make_config(T, 64, E, k, 64, capacity_override=C, dtype='bf16', priority='score')
    ws = moe.workspace(cfg, DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    slot = torch.empty(T, k, dtype=torch.int32, device=DEV)
    dropped = torch.empty(T, k, dtype=torch.uint8, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    rt = torch.full((E, C), -1, dtype=torch.int32, device=DEV)
    w = synth.Workload('s', T=T, d=64, E=E, k=k, d_ff=8, act='gelu', score='softmax', renormalize=-1, cf=1.0,
                       dtype='bf16', seed=5)
    x = synth.to_torch(synth.router_inputs(w)['x'], DEV)
    xe = torch.zeros(E, C, 64, dtype=x.dtype, device=DEV)
    moe.moe_dispatch_by_score(cfg, x, d_idx, torch.from_numpy(g).to(DEV), slot, dropped, counts, rt, xe, ws)
    torch.cuda.synchronize()
    assert dropped_r.any()
    np.testing.assert_array_equal(np_of(counts), counts_r)
    np.testing.assert_array_equal(np_of(slot), slot_r)
    np.testing.assert_array_equal(np_of(dropped).astype(bool), dropped_r)
    np.testing.assert_array_equal(np_of(rt), rt_r)
    # the copy of the kept rows
    xn, xen = np_of(x), np_of(xe)
    kept = np.minimum(counts_r, C)
    for e in range(E):
        np.testing.assert_array_equal(xen[e, :kept[e]], xn[rt_r[e, :kept[e]]])


SCORE_FORWARDS = [('tiny_f32', dict(capacity_override=20)), ('switch_top1_skewed', dict()),
                  ('deepseekmoe_fine', dict(capacity_override=900)), ('mixtral_8x_top2', dict(capacity_override=1800)),
                  ('sigmoid_stress', dict(capacity_override=2500))]


@pytest.mark.parametrize('case', SCORE_FORWARDS, ids=lambda c: c[0])
def test_forward_score_priority(moe, case):
    name, over = case
    w = synth.WORKLOADS[name]
    rows = None
    if w.T > 5000:
        rows = np.sort(np.random.default_rng(6).choice(w.T, 160, replace=False))
    cfg, out, ref = _compare_forward(moe, w, rows=rows, priority='score', **over)
    assert ref['dropped'].any()


# ----------------------------------------------------------------------------- graph capture
@pytest.mark.parametrize('over', [dict(), dict(priority='score', capacity_override=900), dict(routing='expert'),
                                  dict(dropless=True)], ids=['rank', 'score', 'expert_choice', 'dropless'])
def test_forward_replays_from_a_captured_graph(moe, over):
    """moe_forward enqueues kernels only (no memset, copy or allocation), so
    it can be captured into a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager call bit for bit."""
    w = synth.WORKLOADS['deepseekmoe_fine'].with_(T=3000, name='graph')
    say('graph capture', over)
    inp, ex, sh, dev = device_layer(w, moe)
    cfg = moe.config_from_workload(w, **over)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    ref = moe.alloc_outputs(cfg, DEV, logits=True, probs=True, lse=True)
    ws_ref = moe.workspace(cfg, DEV)
    moe.moe_forward(cfg, weights, dev['x'], ref, ws_ref)
    torch.cuda.synchronize()
    out = moe.alloc_outputs(cfg, DEV, logits=True, probs=True, lse=True)
    ws = moe.workspace(cfg, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                         # warm the stream once outside capture
        moe.moe_forward(cfg, weights, dev['x'], out, ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward(cfg, weights, dev['x'], out, ws, stream=s)
    for rep in range(3):
        for t in out.values():                         # scribble between replays
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kk in ref:
            if over.get('routing') == 'expert' and kk in ('slot', 'dropped'):
                continue                               # not written under expert choice
            assert torch.equal(out[kk], ref[kk]), (rep, kk)


# ----------------------------------------------------------------------------- split-k down projection
@pytest.mark.parametrize('act', ['gelu', 'swiglu'])
def test_forward_with_split_k_down_projection(moe, act):
    """Few experts' rows and a narrow model leave the down projection with
    too few tiles to fill the GPU; moe_forward then splits its k range (here
    4 tiles, d_ff 2048 -> 4 parts of 512) and sums the float32 parts in order
    with the bias.  The layer still matches the oracle."""
    w = synth.Workload('sk', T=300, d=256, E=4, k=1, d_ff=2048, act=act, score='softmax', renormalize=-1,
                       cf=1.0, dtype='bf16', seed=71)
    cfg, out, ref = _compare_forward(moe, w)
    assert ref['dropped'].any() or ref['capacity'] * w.E >= w.T
