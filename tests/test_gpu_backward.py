"""Parity of the HIP backward pass (through the C ABI) with the oracle's
chain rule, on an MI355X.

The GPU forward pass runs first (its outputs and workspace feed the backward
pass); the oracle runs its own forward pass on the same inputs and its
backward pass on the same dy.  Routing must come out identical on both sides
for the comparison to be meaningful (the layers below have no near ties).
Bar: every gradient within 2e-2 max-relative of the oracle's (the bf16 bar:
the gradients flow through bf16-stored activations, expert outputs and
gradient rows, each a rounding the oracle does not make).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import backward as B
from oracle import moe as O

from gpu_helpers import DEV, device_layer, f64_of, maxrel, np_of, record

pytestmark = pytest.mark.gpu

ALPHA_AUX, ALPHA_Z = 0.37, 0.11
TOL = 2e-2


@pytest.fixture(scope='module')
def moe():
    assert torch.cuda.is_available(), 'GPU tests need a GPU'
    import mixture_experts_layer_20_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _layer(moe, w, seed):
    inp, ex, sh, dev = device_layer(w, moe)
    rng = np.random.default_rng(seed)
    if w.act == 'gelu':                                   # non-zero biases, bf16-exact
        for kk in ('b_in', 'b_out'):
            bits = synth.bf16_bits((0.1 * rng.standard_normal(ex[kk].shape)).astype(np.float32))
            ex[kk] = bits
            dev[kk] = synth.to_torch(bits, DEV)
    if sh is not None:
        bits = synth.bf16_bits((0.1 * rng.standard_normal(sh['b_in'].shape)).astype(np.float32))
        sh['b_in'] = bits
        dev['bs_in'] = synth.to_torch(np.concatenate(list(bits)), DEV)
    dy = synth.bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
    return inp, ex, sh, dev, dy


def _run(moe, w, seed=0, **over):
    inp, ex, sh, dev, dy = _layer(moe, w, seed)
    cfg = moe.config_from_workload(w, **over)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d, T = w.E, w.d_ff, w.d, w.T
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(T, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dlogit_bias=torch.empty(E, device=DEV), dw_in=torch.empty(E, F, d, dtype=bf, device=DEV),
                 dw_out=torch.empty(E, d, F, dtype=bf, device=DEV), db_out=None, db_in=None,
                 dgates=torch.empty(T, w.k, device=DEV), dlogits=torch.empty(T, E, device=DEV))
    if w.act == 'swiglu':
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device=DEV)
    else:
        grads['db_in'] = torch.empty(E, F, dtype=bf, device=DEV)
        grads['db_out'] = torch.empty(E, d, dtype=bf, device=DEV)
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device=DEV), dws_out=torch.empty(d, fs, dtype=bf, device=DEV),
                     dbs_in=torch.empty(fs, dtype=bf, device=DEV), dbs_out=torch.empty(d, dtype=bf, device=DEV))
    bws = moe.backward_workspace(cfg, DEV)
    dy_t = synth.to_torch(dy, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, dy_t, grads, bws, ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    # the oracle on the same inputs
    dout = 'zero' if over.get('dropped_output') == 'zero' else 'residual'
    ov = over.get('capacity_override', 0)
    fwd = O.moe_forward(w, inp, ex, sh, capacity_override=ov, dropped_output=dout,
                        dropless=bool(over.get('dropless', False)), priority=over.get('priority', 'rank'))
    assert (np_of(out['idx']) == fwd['idx']).all(), 'routing differs from the oracle: pick another seed'
    np.testing.assert_array_equal(np_of(out['slot']), fwd['slot'])
    ref = B.moe_backward(w, inp, ex, sh, fwd, synth.as_f32(dy), ALPHA_AUX, ALPHA_Z, dropped_output=dout)
    return grads, ref, fwd


def _check(name, got, ref):
    err = maxrel(got, ref)
    say(f'  {name}: max-rel {err:.2e}')
    record(name.split('[')[0].split(' (')[0], err)
    assert err <= TOL, (name, err)


def _compare(w, grads, ref):
    _check('dgates', np_of(grads['dgates']), ref['dgates'])
    _check('dlogits', np_of(grads['dlogits']), ref['dz'])
    _check('dx', f64_of(grads['dx']), ref['dx'])
    _check('dw_router', np_of(grads['dw_router']), ref['dw_router'])
    _check('dlogit_bias', np_of(grads['dlogit_bias']), ref['dlogit_bias'])
    ex = ref['experts']
    if w.act == 'swiglu':
        _check('dw_gate', f64_of(grads['dw_gate']), np.stack([g['w_gate'] for g in ex]))
        _check('dw_up', f64_of(grads['dw_in']), np.stack([g['w_up'] for g in ex]))
    else:
        _check('dw_in', f64_of(grads['dw_in']), np.stack([g['w_in'] for g in ex]))
        _check('db_in', f64_of(grads['db_in']), np.stack([g['b_in'] for g in ex]))
        _check('db_out', f64_of(grads['db_out']), np.stack([g['b_out'] for g in ex]))
    _check('dw_out', f64_of(grads['dw_out']), np.stack([g['w_out'] for g in ex]))
    if w.n_shared:
        sg = ref['shared']
        _check('dws_in', f64_of(grads['dws_in']), np.concatenate([g['w_in'] for g in sg], 0))
        _check('dws_out', f64_of(grads['dws_out']), np.concatenate([g['w_out'] for g in sg], 1))
        _check('dbs_in', f64_of(grads['dbs_in']), np.concatenate([g['b_in'] for g in sg]))
        _check('dbs_out', f64_of(grads['dbs_out']), sg[0]['b_out'])


BWD_CASES = [
    ('gelu_renorm_drops', synth.Workload('ba', T=700, d=256, E=8, k=2, d_ff=384, act='gelu', score='softmax',
                                         renormalize=-1, cf=1.0, dtype='bf16', seed=61), {}),
    ('swiglu_renorm', synth.Workload('bb', T=600, d=256, E=4, k=2, d_ff=512, act='swiglu', score='softmax',
                                     renormalize=-1, cf=1.25, dtype='bf16', seed=62), {}),
    ('sigmoid_shared', synth.Workload('bc', T=500, d=128, E=16, k=3, d_ff=128, act='gelu', score='sigmoid',
                                      renormalize=1, cf=1.0, dtype='bf16', seed=63, select_bias=True, n_shared=2,
                                      d_ff_shared=128), {}),
    ('top1_raw_fallback', synth.Workload('bd', T=1000, d=128, E=16, k=1, d_ff=256, act='gelu', score='softmax',
                                         renormalize=-1, cf=1.0, dtype='bf16', seed=64,
                                         logit_bias='first_two_plus2'), {}),
    ('zero_fallback_swiglu', synth.Workload('be', T=300, d=128, E=4, k=2, d_ff=256, act='swiglu',
                                            score='softmax', renormalize=-1, cf=1.0, dtype='bf16', seed=65),
     dict(capacity_override=40, dropped_output='zero')),
    ('sigmoid_raw_ragged', synth.Workload('bf', T=333, d=64, E=8, k=2, d_ff=72, act='gelu', score='sigmoid',
                                          renormalize=0, cf=1.25, dtype='bf16', seed=66), {}),
    # SwiGLU width not a multiple of the 64-k stage: the input gradient takes
    # the transposed [W_gate; W_up] copy instead of the two k-major matrices
    ('swiglu_width_off_stage', synth.Workload('bh', T=300, d=64, E=4, k=2, d_ff=200, act='swiglu',
                                              score='softmax', renormalize=-1, cf=1.25, dtype='bf16', seed=69), {}),
    # an expert no token picks: its rows are empty, so the k-major weight
    # gradients contract over nothing (exact zeros), SwiGLU and GELU
    ('empty_expert_swiglu', synth.Workload('bi', T=400, d=128, E=8, k=2, d_ff=128, act='swiglu', score='softmax',
                                           renormalize=-1, cf=1.25, dtype='bf16', seed=67,
                                           logit_bias='last_minus30'), {}),
    ('empty_expert_gelu_dropless', synth.Workload('bj', T=400, d=128, E=8, k=2, d_ff=192, act='gelu',
                                                  score='softmax', renormalize=-1, cf=1.25, dtype='bf16', seed=67,
                                                  logit_bias='last_minus30'), dict(dropless=True)),
    # more experts than 16-byte column chunks of a row (E > d/8): the input
    # gradient's router term reads dL/dz of every expert from every lane
    ('narrow_rows_many_experts', synth.Workload('bg', T=256, d=64, E=48, k=4, d_ff=64, act='gelu',
                                                score='softmax', renormalize=-1, cf=1.0, dtype='bf16', seed=68), {}),
    # the configuration's limits: 256 experts (four per lane in the router
    # backward, 256 expert groups in the GEMMs) and 32 choices per token;
    # seeds whose 32nd and 33rd keys are at least 3e-5 apart, so that both
    # sides route alike
    ('limits_E256_k32', synth.Workload('bl', T=300, d=64, E=256, k=32, d_ff=64, act='gelu', score='softmax',
                                       renormalize=-1, cf=1.25, dtype='bf16', seed=49), {}),
    ('limits_E256_k32_sigmoid_dropless', synth.Workload('bm', T=300, d=64, E=256, k=32, d_ff=64, act='gelu',
                                                        score='sigmoid', renormalize=1, cf=1.25, dtype='bf16',
                                                        seed=41, select_bias=True), dict(dropless=True)),
]


def test_backward_gives_an_empty_expert_zero_weight_gradients(moe):
    name, w, over = [c for c in BWD_CASES if c[0] == 'empty_expert_swiglu'][0]
    grads, ref, fwd = _run(moe, w, seed=3, **over)
    assert not (fwd['idx'] == w.E - 1).any()
    for kk in ('dw_gate', 'dw_in', 'dw_out'):
        assert not np_of(grads[kk])[w.E - 1].any(), kk          # exactly zero
    _compare(w, grads, ref)


@pytest.mark.parametrize('case', BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_parity(moe, case):
    name, w, over = case
    say('backward', name)
    grads, ref, fwd = _run(moe, w, **over)
    if name in ('gelu_renorm_drops', 'top1_raw_fallback', 'zero_fallback_swiglu'):
        assert fwd['dropped'].any()
    _compare(w, grads, ref)
    if name == 'top1_raw_fallback':
        # fully dropped tokens pass dy through (plus their router term)
        assert (~(~fwd['dropped']).any(axis=1)).any()


@pytest.mark.parametrize('priority', ['token', 'score'])
def test_backward_capacity_priorities(moe, priority):
    """The backward pass reads the forward's slots and drops whatever queue
    order decided them: token-major and batch-prioritised (score) capacity."""
    name, w, over = BWD_CASES[0]
    say('backward priority', priority)
    grads, ref, fwd = _run(moe, w, priority=priority)
    assert fwd['dropped'].any()
    _compare(w, grads, ref)


def test_backward_single_token(moe):
    w = synth.Workload('bz', T=1, d=64, E=4, k=2, d_ff=64, act='gelu', score='softmax', renormalize=-1, cf=1.0,
                       dtype='bf16', seed=67)
    grads, ref, fwd = _run(moe, w)
    _compare(w, grads, ref)


FULL = ['mixtral_8x_top2', 'deepseekmoe_fine', 'sigmoid_stress', 'switch_top1_skewed']


@pytest.mark.parametrize('name', FULL)
def test_backward_full_size_sampled(moe, name):
    """The workloads at full size: the gate, logit and input gradients of 48
    sampled tokens (and the extreme-logit and duplicated rows of the stress
    layer), and sampled rows/columns of the expert weight gradients (each a
    sum over all of an expert's kept rows), against the oracle computed for
    just those."""
    w = synth.WORKLOADS[name]
    say('backward full size', name)
    inp, ex, sh, dev = device_layer(w, moe)
    rng = np.random.default_rng(9)
    dy = synth.bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
    cfg = moe.config_from_workload(w)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d, T, k = w.E, w.d_ff, w.d, w.T, w.k
    glu = w.act == 'swiglu'
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(T, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dw_in=torch.empty(E, F, d, dtype=bf, device=DEV), dw_out=torch.empty(E, d, F, dtype=bf, device=DEV),
                 dgates=torch.empty(T, k, device=DEV), dlogits=torch.empty(T, E, device=DEV))
    if glu:
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device=DEV)
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device=DEV), dws_out=torch.empty(d, fs, dtype=bf, device=DEV))
    bws = moe.backward_workspace(cfg, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, synth.to_torch(dy, DEV), grads, bws, ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    rows = rng.choice(T, 48, replace=False)
    if name == 'sigmoid_stress':
        rows = np.concatenate([rows, inp['extreme_rows'][:8], inp['dup_rows'][:8]])
    rows = np.unique(rows)
    get = (lambda e: {kk: v[e] for kk, v in ex.items()})
    gsh = None if sh is None else (lambda s_: {kk: v[s_] for kk, v in sh.items()})
    fwd = O.moe_forward(w, inp, get, gsh, rows=rows)
    # tokens whose choices or drops came out differently (near-tie keys, see
    # the forward parity rules) are left out, and so are the experts whose
    # kept rows differ; there must be few
    gi, gd = np_of(out['idx']), np_of(out['dropped']).astype(bool)
    same = (gi == fwd['idx']).all(axis=1) & (gd == fwd['dropped']).all(axis=1)
    assert same.mean() > 0.999, int((~same).sum())
    rows = rows[same[rows]]
    x = synth.as_f32(inp['x']).astype(np.float64)
    dyf = synth.as_f32(dy).astype(np.float64)
    kept = ~fwd['dropped']
    wts = [{kk: synth.as_f32(v).astype(np.float64) for kk, v in get(e).items()} for e in range(E)]
    swts = [{kk: synth.as_f32(v).astype(np.float64) for kk, v in gsh(s_).items()} for s_ in range(w.n_shared)]
    # per sampled token: gate gradients, its experts' input gradients, dz and dx
    dg = np.zeros((rows.size, k))
    dxe = np.zeros((rows.size, d))
    for i, t in enumerate(rows):
        for j in range(k):
            if not kept[t, j]:
                continue
            e = fwd['idx'][t, j]
            _, o = O.expert_ffn(x[t][None], wts[e], w.act, 'bf16')
            dg[i, j] = float((dyf[t] * o[0]).sum())
            da, _ = B.expert_ffn_backward(x[t][None], wts[e], w.act, 'bf16', fwd['gates'][t, j] * dyf[t][None])
            dxe[i] += da[0]
        for sw in swts:
            da, _ = B.expert_ffn_backward(x[t][None], sw, 'gelu', 'bf16', dyf[t][None])
            dxe[i] += da[0]
        if not swts and not kept[t].any():
            dxe[i] += dyf[t]                                 # residual fallback
    counts = np.bincount(fwd['idx'].ravel(), minlength=E)
    dz = B.router_backward(fwd['logits'][rows], fwd['idx'][rows], dg, w.score, w.renormalize, counts / (T * k),
                           ALPHA_AUX, ALPHA_Z, n_tokens=T)
    dx = dxe + dz @ np.asarray(inp['w_router'], np.float64).T
    _check('dgates (sampled tokens)', np_of(grads['dgates'])[rows], dg)
    _check('dlogits (sampled tokens)', np_of(grads['dlogits'])[rows], dz)
    _check('dx (sampled tokens)', f64_of(grads['dx'])[rows], dx)
    # weight gradients: for expert e and hidden unit f, over all its kept rows
    g_in, g_out = f64_of(grads['dw_in']), f64_of(grads['dw_out'])
    g_gate = f64_of(grads['dw_gate']) if glu else None
    for e, f in [(0, 5), (E - 1, F - 1), (E // 2, F // 3)]:
        t_e, j_e = np.nonzero((fwd['idx'] == e) & kept)
        if t_e.size == 0 or set(t_e.tolist()) != set(np.nonzero(((gi == e) & ~gd).any(axis=1))[0].tolist()):
            continue
        a = x[t_e]
        d_out = fwd['gates'][t_e, j_e][:, None] * dyf[t_e]
        dh = d_out @ wts[e]['w_out'][:, f]
        if glu:
            gp = a @ wts[e]['w_gate'][f]
            up = a @ wts[e]['w_up'][f]
            h = O.round_store(O.silu(gp) * up, 'bf16')
            _check(f'dw_up[{e}][{f}]', g_in[e][f], (dh * O.silu(gp)) @ a)
            _check(f'dw_gate[{e}][{f}]', g_gate[e][f], (dh * up * B.silu_grad(gp)) @ a)
        else:
            u = a @ wts[e]['w_in'][f] + (wts[e]['b_in'][f] if wts[e].get('b_in') is not None else 0.0)
            h = O.round_store(O.gelu(u), 'bf16')
            _check(f'dw_in[{e}][{f}]', g_in[e][f], (dh * B.gelu_grad(u)) @ a)
        _check(f'dw_out[{e}][:, {f}]', g_out[e][:, f], d_out.T @ h)

def _gpu_pass(moe, w, dev, dy, k_grads=None, **over):
    cfg = moe.config_from_workload(w, **over)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d, T = w.E, w.d_ff, w.d, w.T
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(T, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dw_in=torch.empty(E, F, d, dtype=bf, device=DEV), dw_out=torch.empty(E, d, F, dtype=bf, device=DEV),
                 dgates=torch.empty(T, k_grads or w.k, device=DEV), dlogits=torch.empty(T, E, device=DEV))
    if w.act == 'swiglu':
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device=DEV)
    else:
        grads['db_in'] = torch.empty(E, F, dtype=bf, device=DEV)
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device=DEV), dws_out=torch.empty(d, fs, dtype=bf, device=DEV))
    bws = moe.backward_workspace(cfg, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, synth.to_torch(dy, DEV), grads, bws, ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    return out, grads


@pytest.mark.parametrize('case', [c for c in BWD_CASES if c[0] in ('gelu_renorm_drops', 'swiglu_renorm',
                                                                   'sigmoid_shared')], ids=lambda c: c[0])
def test_saved_preactivations_equal_recomputation(moe, case):
    """With save_preact the forward pass keeps the expert (and shared)
    pre-activations and the backward pass reads them instead of recomputing:
    the forward outputs and every gradient are bit-identical either way (the
    same products summed in the same order)."""
    name, w, over = case
    say('save_preact', name)
    inp, ex, sh, dev, dy = _layer(moe, w, 0)
    out0, g0 = _gpu_pass(moe, w, dev, dy, **over)
    out1, g1 = _gpu_pass(moe, w, dev, dy, save_preact=True, **over)
    for kk in out0:
        assert torch.equal(out0[kk], out1[kk]), kk
    for kk in g0:
        assert torch.equal(g0[kk], g1[kk]), kk


@pytest.mark.parametrize('case', [c for c in BWD_CASES if c[0] in ('gelu_renorm_drops', 'swiglu_renorm', 'sigmoid_shared',
                                                                   'sigmoid_raw_ragged')], ids=lambda c: c[0])
def test_backward_dropless(moe, case):
    """Dropless mode: every choice kept in packed rows; the expert GEMMs run on
    the packed rows and the weight gradients contract over each expert's own
    row count (reached through per-expert row lists)."""
    name, w, over = case
    say('backward dropless', name)
    grads, ref, fwd = _run(moe, w, dropless=True)
    assert not fwd['dropped'].any()
    _compare(w, grads, ref)


@pytest.mark.parametrize('name', ['deepseekmoe_fine', 'swiglu_tail'])
def test_saved_preactivations_equal_recomputation_with_a_split_last_round(moe, name):
    # the 64-expert layer at full size, and a SwiGLU layer of 8 experts filled
    # to 9 row tiles whose gate/up launch (d = 4096, 8 x 9 x 8 = 576 tiles)
    # splits its last round of 64 tiles along k: the backward's recomputation
    # repeats the forward's launch, so saved and recomputed pre-activations,
    # and every gradient, are the same bits
    if name == 'deepseekmoe_fine':
        w, over = synth.WORKLOADS['deepseekmoe_fine'], {}
    else:
        w = synth.Workload('swiglu_tail', T=12000, d=4096, E=8, k=2, d_ff=1024, act='swiglu', score='softmax',
                           renormalize=-1, cf=1.25, dtype='bf16', seed=66)
        over = dict(capacity_override=2304)
    say('save_preact with a split last round', name)
    inp, ex, sh, dev, dy = _layer(moe, w, 0)
    out0, g0 = _gpu_pass(moe, w, dev, dy, **over)
    out1, g1 = _gpu_pass(moe, w, dev, dy, save_preact=True, **over)
    for kk in out0:
        assert torch.equal(out0[kk], out1[kk]), kk
    for kk in g0:
        assert torch.equal(g0[kk], g1[kk]), kk


def test_saved_preactivations_equal_recomputation_dropless(moe):
    name, w, over = BWD_CASES[1]
    inp, ex, sh, dev, dy = _layer(moe, w, 0)
    out0, g0 = _gpu_pass(moe, w, dev, dy, dropless=True)
    out1, g1 = _gpu_pass(moe, w, dev, dy, dropless=True, save_preact=True)
    for kk in out0:
        assert torch.equal(out0[kk], out1[kk]), kk
    for kk in g0:
        assert torch.equal(g0[kk], g1[kk]), kk


# ----------------------------------------------------------------------------- expert choice
EC_BWD_CASES = [
    ('ec_gelu_fallback', synth.Workload('ea', T=600, d=128, E=8, k=2, d_ff=256, act='gelu', score='softmax',
                                        renormalize=-1, cf=1.0, dtype='bf16', seed=71), {}),
    ('ec_swiglu_sigmoid', synth.Workload('eb', T=400, d=256, E=16, k=2, d_ff=128, act='swiglu', score='sigmoid',
                                         renormalize=1, cf=1.25, dtype='bf16', seed=72), {}),
    ('ec_gelu_shared', synth.Workload('ec', T=300, d=128, E=8, k=2, d_ff=128, act='gelu', score='softmax',
                                      renormalize=-1, cf=1.0, dtype='bf16', seed=73, n_shared=1,
                                      d_ff_shared=128), {}),
    ('ec_zero_fallback', synth.Workload('ed', T=256, d=64, E=4, k=1, d_ff=64, act='gelu', score='softmax',
                                        renormalize=-1, cf=1.0, dtype='bf16', seed=74),
     dict(capacity_override=24, dropped_output='zero')),
    ('ec_wide_160', synth.Workload('ee', T=320, d=64, E=160, k=4, d_ff=64, act='gelu', score='softmax',
                                   renormalize=-1, cf=1.0, dtype='bf16', seed=75), {}),
    ('ec_all_tokens', synth.Workload('ef', T=40, d=64, E=4, k=2, d_ff=64, act='swiglu', score='softmax',
                                     renormalize=-1, cf=1.0, dtype='bf16', seed=76), dict(capacity_override=64)),
]


def _run_ec(moe, w, seed=0, **over):
    """GPU forward + backward under expert choice, and the oracle's forward and
    backward on the same inputs; the picks must come out identical."""
    inp, ex, sh, dev, dy = _layer(moe, w, seed)
    cfg = moe.config_from_workload(w, routing='expert', **over)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d, T = w.E, w.d_ff, w.d, w.T
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(T, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dlogit_bias=torch.empty(E, device=DEV), dw_in=torch.empty(E, F, d, dtype=bf, device=DEV),
                 dw_out=torch.empty(E, d, F, dtype=bf, device=DEV), db_out=None, db_in=None,
                 dgates=torch.empty(T, E, device=DEV), dlogits=torch.empty(T, E, device=DEV))
    if w.act == 'swiglu':
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device=DEV)
    else:
        grads['db_in'] = torch.empty(E, F, dtype=bf, device=DEV)
        grads['db_out'] = torch.empty(E, d, dtype=bf, device=DEV)
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device=DEV), dws_out=torch.empty(d, fs, dtype=bf, device=DEV),
                     dbs_in=torch.empty(fs, dtype=bf, device=DEV), dbs_out=torch.empty(d, dtype=bf, device=DEV))
    bws = moe.backward_workspace(cfg, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, synth.to_torch(dy, DEV), grads, bws, ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    dout = 'zero' if over.get('dropped_output') == 'zero' else 'residual'
    fwd = O.moe_forward(w, inp, ex, sh, capacity_override=over.get('capacity_override', 0), dropped_output=dout,
                        routing='expert')
    np.testing.assert_array_equal(np_of(out['sel']), fwd['sel'], 'picks differ from the oracle: pick another seed')
    ref = B.moe_backward_expert_choice(w, inp, ex, sh, fwd, synth.as_f32(dy), ALPHA_AUX, ALPHA_Z,
                                       dropped_output=dout)
    return out, grads, ref, fwd


@pytest.mark.parametrize('case', EC_BWD_CASES, ids=[c[0] for c in EC_BWD_CASES])
def test_backward_expert_choice_parity(moe, case):
    """Expert choice: the gate of a pick is the router probability, so dprobs
    [T,E] (0 where not picked) reaches the logits through the probabilities'
    Jacobian; unpicked tokens pass dy to dx unless shared experts or the zero
    output take their place."""
    name, w, over = case
    say('backward expert choice', name)
    out, grads, ref, fwd = _run_ec(moe, w, **over)
    picked = (fwd['sel'] >= 0)
    if name in ('ec_gelu_fallback', 'ec_zero_fallback'):
        assert (~picked.any(axis=1)).any()                 # tokens no expert picked
    if name == 'ec_all_tokens':
        assert picked.all()
    dp = np_of(grads['dgates'])
    assert (dp[~picked] == 0).all()
    _check('dprobs', dp, ref['dprobs'])
    _check('dlogits', np_of(grads['dlogits']), ref['dz'])
    _check('dx', f64_of(grads['dx']), ref['dx'])
    _check('dw_router', np_of(grads['dw_router']), ref['dw_router'])
    _check('dlogit_bias', np_of(grads['dlogit_bias']), ref['dlogit_bias'])
    ex = ref['experts']
    if w.act == 'swiglu':
        _check('dw_gate', f64_of(grads['dw_gate']), np.stack([g['w_gate'] for g in ex]))
        _check('dw_up', f64_of(grads['dw_in']), np.stack([g['w_up'] for g in ex]))
    else:
        _check('dw_in', f64_of(grads['dw_in']), np.stack([g['w_in'] for g in ex]))
        _check('db_in', f64_of(grads['db_in']), np.stack([g['b_in'] for g in ex]))
        _check('db_out', f64_of(grads['db_out']), np.stack([g['b_out'] for g in ex]))
    _check('dw_out', f64_of(grads['dw_out']), np.stack([g['w_out'] for g in ex]))
    if w.n_shared:
        sg = ref['shared']
        _check('dws_in', f64_of(grads['dws_in']), np.concatenate([g['w_in'] for g in sg], 0))
        _check('dws_out', f64_of(grads['dws_out']), np.concatenate([g['w_out'] for g in sg], 1))


def test_backward_expert_choice_saved_preactivations(moe):
    name, w, over = EC_BWD_CASES[2]
    inp, ex, sh, dev, dy = _layer(moe, w, 0)
    out0, g0 = _gpu_pass(moe, w, dev, dy, routing='expert', k_grads=w.E)
    out1, g1 = _gpu_pass(moe, w, dev, dy, routing='expert', k_grads=w.E, save_preact=True)
    for kk in out0:
        if kk not in ('slot', 'dropped'):                 # not written under expert choice
            assert torch.equal(out0[kk], out1[kk]), kk
    for kk in g0:
        assert torch.equal(g0[kk], g1[kk]), kk


@pytest.mark.parametrize('name', ['mixtral_8x_top2', 'deepseekmoe_fine', 'sigmoid_stress'])
def test_backward_expert_choice_full_size_sampled(moe, name):
    """Expert choice at full size: the probability, logit and input gradients
    of 48 sampled tokens, and sampled rows/columns of the expert weight
    gradients (sums over all of an expert's picks), against the oracle
    computed for just those.  Tokens whose picks differ from the oracle's
    (probabilities within rounding of an expert's n-th largest) and experts
    whose pick sets differ are left out; there must be few."""
    w = synth.WORKLOADS[name]
    say('backward expert choice full size', name)
    inp, ex, sh, dev = device_layer(w, moe)
    rng = np.random.default_rng(19)
    dy = synth.bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32))
    cfg = moe.config_from_workload(w, routing='expert')
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d, T = w.E, w.d_ff, w.d, w.T
    glu = w.act == 'swiglu'
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(T, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dw_in=torch.empty(E, F, d, dtype=bf, device=DEV), dw_out=torch.empty(E, d, F, dtype=bf, device=DEV),
                 dgates=torch.empty(T, E, device=DEV), dlogits=torch.empty(T, E, device=DEV))
    if glu:
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device=DEV)
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device=DEV), dws_out=torch.empty(d, fs, dtype=bf, device=DEV))
    bws = moe.backward_workspace(cfg, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, synth.to_torch(dy, DEV), grads, bws, ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    rows = np.unique(rng.choice(T, 48, replace=False))
    get = (lambda e: {kk: v[e] for kk, v in ex.items()})
    gsh = None if sh is None else (lambda s_: {kk: v[s_] for kk, v in sh.items()})
    fwd = O.moe_forward(w, inp, get, gsh, rows=rows, routing='expert')
    gsel = np_of(out['sel'])
    gp, rp = gsel >= 0, fwd['sel'] >= 0
    same = (gp == rp).all(axis=1)
    assert same.mean() > 0.995, int((~same).sum())
    rows = rows[same[rows]]
    p = np.asarray(fwd['probs'], np.float64)
    x = synth.as_f32(inp['x']).astype(np.float64)
    dyf = synth.as_f32(dy).astype(np.float64)
    wts = [{kk: synth.as_f32(v).astype(np.float64) for kk, v in get(e).items()} for e in range(E)]
    swts = [{kk: synth.as_f32(v).astype(np.float64) for kk, v in gsh(s_).items()} for s_ in range(w.n_shared)]
    dp = np.zeros((rows.size, E))
    dxe = np.zeros((rows.size, d))
    for i, t in enumerate(rows):
        for e in np.nonzero(rp[t])[0]:
            _, o = O.expert_ffn(x[t][None], wts[e], w.act, 'bf16')
            dp[i, e] = float((dyf[t] * o[0]).sum())
            da, _ = B.expert_ffn_backward(x[t][None], wts[e], w.act, 'bf16', p[t, e] * dyf[t][None])
            dxe[i] += da[0]
        for sw in swts:
            da, _ = B.expert_ffn_backward(x[t][None], sw, 'gelu', 'bf16', dyf[t][None])
            dxe[i] += da[0]
        if not swts and not rp[t].any():
            dxe[i] += dyf[t]                                 # residual fallback
    counts = rp.sum(axis=0).astype(np.float64)
    v = ALPHA_AUX * E * (counts / counts.sum()) / T
    z = np.asarray(fwd['logits'], np.float64)[rows]
    dz = B.probs_backward(z, dp + v[None, :], w.score)
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    dz += ALPHA_Z * 2.0 * lse[:, None] * O.softmax(z) / T
    dx = dxe + dz @ np.asarray(inp['w_router'], np.float64).T
    _check('dprobs (sampled tokens)', np_of(grads['dgates'])[rows], dp)
    _check('dlogits (sampled tokens)', np_of(grads['dlogits'])[rows], dz)
    _check('dx (sampled tokens)', f64_of(grads['dx'])[rows], dx)
    g_in, g_out = f64_of(grads['dw_in']), f64_of(grads['dw_out'])
    g_gate = f64_of(grads['dw_gate']) if glu else None
    checked = 0
    for e, f in [(0, 5), (E - 1, F - 1), (E // 2, F // 3)]:
        if not (gp[:, e] == rp[:, e]).all():
            continue
        checked += 1
        t_e = np.nonzero(rp[:, e])[0]
        a = x[t_e]
        d_out = p[t_e, e][:, None] * dyf[t_e]
        dh = d_out @ wts[e]['w_out'][:, f]
        if glu:
            gpre = a @ wts[e]['w_gate'][f]
            up = a @ wts[e]['w_up'][f]
            h = O.round_store(O.silu(gpre) * up, 'bf16')
            _check(f'dw_up[{e}][{f}]', g_in[e][f], (dh * O.silu(gpre)) @ a)
            _check(f'dw_gate[{e}][{f}]', g_gate[e][f], (dh * up * B.silu_grad(gpre)) @ a)
        else:
            u = a @ wts[e]['w_in'][f] + (wts[e]['b_in'][f] if wts[e].get('b_in') is not None else 0.0)
            h = O.round_store(O.gelu(u), 'bf16')
            _check(f'dw_in[{e}][{f}]', g_in[e][f], (dh * B.gelu_grad(u)) @ a)
        _check(f'dw_out[{e}][:, {f}]', g_out[e][:, f], d_out.T @ h)
    assert checked > 0


@pytest.mark.parametrize('over', [dict(), dict(save_preact=True), dict(routing='expert')],
                         ids=['recompute', 'save_preact', 'expert_choice'])
def test_training_step_replays_from_a_captured_graph(moe, over):
    """moe_forward followed by moe_backward enqueues kernels only (zero fills
    are kernels), so a whole training step of the layer captures into one HIP
    graph: every replay, with eager scribbling and synchronisations between
    replays, gives the eager call's outputs and gradients bit for bit."""
    name, w, _ = BWD_CASES[2]                          # sigmoid scores, shared experts
    say('graph capture of forward + backward', over)
    inp, ex, sh, dev, dy = _layer(moe, w, 0)
    ec = over.get('routing') == 'expert'
    out0, g0 = _gpu_pass(moe, w, dev, dy, k_grads=w.E if ec else None, **over)
    cfg = moe.config_from_workload(w, **over)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    grads = {kk: torch.empty_like(v) for kk, v in g0.items()}
    bws = moe.backward_workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    dy_t = synth.to_torch(dy, DEV)
    s = torch.cuda.Stream()

    def step():
        moe.moe_forward(cfg, weights, dev['x'], out, ws, stream=s)
        moe.moe_backward(cfg, weights, dev['x'], out, ws, dy_t, grads, bws, ALPHA_AUX, ALPHA_Z, stream=s)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                         # warm the stream once outside capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for t in list(out.values()) + list(grads.values()):   # scribble between replays
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kk in out0:
            if ec and kk in ('slot', 'dropped'):
                continue                               # not written under expert choice
            assert torch.equal(out[kk], out0[kk]), (rep, kk)
        for kk in g0:
            assert torch.equal(grads[kk], g0[kk]), (rep, kk)


@pytest.mark.parametrize('routing', ['token', 'expert'])
def test_backward_empty_batch(moe, routing):
    """T = 0: every weight gradient is zero (written, not left as it was)."""
    name, w1, _ = BWD_CASES[2]                         # shared experts, GELU biases
    w = w1.with_(T=0, name='empty')
    inp, ex, sh, dev, dy = _layer(moe, w1.with_(T=1, name='one'), 0)
    dev['x'] = dev['x'][:0]
    cfg = moe.config_from_workload(w, routing=routing)
    out = moe.alloc_outputs(cfg, DEV, logits=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    E, F, d = w.E, w.d_ff, w.d
    fs = w.n_shared * w.d_ff_shared
    bf = torch.bfloat16
    grads = dict(dx=torch.empty(0, d, dtype=bf, device=DEV), dw_router=torch.empty(d, E, device=DEV),
                 dlogit_bias=torch.empty(E, device=DEV), dw_in=torch.empty(E, F, d, dtype=bf, device=DEV),
                 dw_out=torch.empty(E, d, F, dtype=bf, device=DEV), db_in=torch.empty(E, F, dtype=bf, device=DEV),
                 db_out=torch.empty(E, d, dtype=bf, device=DEV), dws_in=torch.empty(fs, d, dtype=bf, device=DEV),
                 dws_out=torch.empty(d, fs, dtype=bf, device=DEV), dbs_in=torch.empty(fs, dtype=bf, device=DEV),
                 dbs_out=torch.empty(d, dtype=bf, device=DEV))
    for t in grads.values():
        t.view(torch.uint8).fill_(0xA5)
    bws = moe.backward_workspace(cfg, DEV)
    moe.moe_backward(cfg, weights, dev['x'], out, ws, torch.empty(0, d, dtype=bf, device=DEV), grads, bws,
                     ALPHA_AUX, ALPHA_Z)
    torch.cuda.synchronize()
    for kk, t in grads.items():
        if t.numel():
            assert (t.float() == 0).all(), kk
