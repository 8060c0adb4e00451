"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
calls through the C ABI, and the comparison rules.

Comparison rules (the bar the tests hold the HIP path to):
  * integer and index outputs (idx, slot, dropped, counts, row_token, stats):
    bit-exact, given identical float32 logits;
  * float32 outputs: max-relative error ||a - b||_inf / ||b||_inf <= 1e-5;
  * bf16 layer output y: max-relative error <= 2e-2;
  * losses: |a - b| / |b| <= 1e-5;
  * end to end (logits computed on both sides): the GPU logits must lie within
    the float32 dot-product error bound of the oracle's; tokens whose ordered
    top-(k+1) keys have an adjacent gap below max(1e-5, what the observed logit
    difference can move a key) are "near-tie" tokens and may route
    differently; probabilities, gates and LSE get the float32 tolerance plus
    the change the observed logit difference propagates into them.
"""
import math

import numpy as np
import torch

import synth
from oracle import moe as O

DEV = 'cuda'


def maxrel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a - b).max())


def np_of(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f64_of(t):
    return synth.as_f32(np_of(t)).astype(np.float64)


def device_layer(w, moe):
    """Router inputs and stacked expert weights of workload w on the GPU."""
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    d = dict(x=synth.to_torch(inp['x'], DEV), w_router=synth.to_torch(inp['w_router'], DEV),
             logit_bias=synth.to_torch(inp['logit_bias'], DEV),
             select_bias=synth.to_torch(inp['select_bias'], DEV))
    for kk, v in ex.items():
        if kk in ('b_in', 'b_out'):
            v = synth.bf16_bits(v) if w.dtype == 'bf16' else v
        d[kk] = synth.to_torch(v, DEV)
    if w.act == 'swiglu':
        d['w_in'] = d.pop('w_up')
    sh = None
    if w.n_shared:
        sh = synth.all_expert_weights(w, shared=True)
        cat_in = np.concatenate(list(sh['w_in']), 0)
        cat_out = np.concatenate(list(sh['w_out']), 1)
        bs_in = np.concatenate(list(sh['b_in']))
        bs_out = sh['b_out'].sum(0).astype(np.float32)
        if w.dtype == 'bf16':
            bs_in, bs_out = synth.bf16_bits(bs_in), synth.bf16_bits(bs_out)
        d.update(ws_in=synth.to_torch(cat_in, DEV), ws_out=synth.to_torch(cat_out, DEV),
                 bs_in=synth.to_torch(bs_in, DEV), bs_out=synth.to_torch(bs_out, DEV))
    return inp, ex, sh, d


def forward(moe, w, dev, **over):
    cfg = moe.config_from_workload(w, **over)
    out = moe.alloc_outputs(cfg, DEV, logits=True, probs=True, lse=True)
    ws = moe.workspace(cfg, DEV)
    weights = {kk: v for kk, v in dev.items() if kk != 'x'}
    moe.moe_forward(cfg, weights, dev['x'], out, ws)
    torch.cuda.synchronize()
    return cfg, out


def logit_error_bound(x, w_router, logit_bias=None):
    """Higham's bound for a float32 dot product in any summation order, plus the
    final rounding: |z - z_ref| <= gamma_d * sum |x w| + u |z_ref| (+ the bias add)."""
    u = 2.0 ** -24
    d = x.shape[1]
    gam = 3 * d * u / (1 - 3 * d * u)          # generous: split or fused products
    S = np.abs(x.astype(np.float64)) @ np.abs(w_router.astype(np.float64))
    if logit_bias is not None:
        S = S + np.abs(logit_bias.astype(np.float64))
    return gam * S


def near_tie_tokens(z_ref, z_gpu, k, score, select_bias):
    """Tokens whose selection may legitimately differ between two float32 logit
    sets: some adjacent gap among the oracle's top-(k+1) keys is below
    max(1e-5, twice the largest key difference the observed logit difference
    can cause, plus a few float32 ulps of the key)."""
    dz = np.abs(np.asarray(z_gpu, np.float64) - np.asarray(z_ref, np.float64)).max(axis=1)
    key = O.selection_keys(z_ref, score, select_bias).astype(np.float64)
    srt = -np.sort(-key, axis=1)
    kk = min(k + 1, key.shape[1])
    if kk < 2:
        return np.zeros(key.shape[0], bool)
    gaps = srt[:, :kk - 1] - srt[:, 1:kk]
    lip = 0.25 if score == 'sigmoid' else 1.0          # sigmoid is 1/4-Lipschitz
    ulps = 8 * 2.0 ** -24 * np.maximum(np.abs(srt[:, 0]), 1.0)
    thr = np.maximum(1e-5, 2 * lip * dz + ulps)
    return (gaps < thr[:, None]).any(axis=1)


def assert_propagated(got, ref, dz, rel=1e-5, what=''):
    """|got - ref| <= rel * max|ref| + |ref| * (exp(2 dz_t) - 1), row-wise: the
    float32 tolerance plus what a logit difference of at most dz_t in row t can
    move a (log-)softmax-derived value (log-softmax is 2-Lipschitz in max norm)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    dzr = np.asarray(dz, np.float64).reshape((-1,) + (1,) * (ref.ndim - 1))
    allowed = rel * np.abs(ref).max() + np.abs(ref) * np.expm1(2 * dzr)
    bad = np.abs(got - ref) > allowed
    assert not bad.any(), (what, np.argwhere(bad)[:5], float((np.abs(got - ref) / np.maximum(allowed, 1e-300)).max()))


def check_capacity_valid(idx, slot, dropped, counts, C, E, priority='rank'):
    """Properties any correct slot assignment has for the given choices."""
    T, k = idx.shape
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    order = [(t, j) for j in range(k) for t in range(T)] if priority == 'rank' else \
        [(t, j) for t in range(T) for j in range(k)]
    nxt = np.zeros(E, np.int64)
    for t, j in order:
        e = idx[t, j]
        assert slot[t, j] == nxt[e]
        nxt[e] += 1
    np.testing.assert_array_equal(dropped, slot >= C)


def check_score_capacity_valid(idx, gates, slot, dropped, counts, C, E):
    """Properties any correct score-priority assignment has for the given
    choices and float32 gates: per expert, min(count, C) kept, no dropped gate
    above a kept one (equal gates: the earlier in the rank-major queue is
    kept), kept numbered 0.. and dropped C.. in queue order."""
    T, k = idx.shape
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    queue = [(t, j) for j in range(k) for t in range(T)]
    per = {e: [] for e in range(E)}
    for t, j in queue:
        per[int(idx[t, j])].append((t, j))
    for e, q in per.items():
        g = np.array([gates[t, j] for t, j in q], np.float32)
        kept = np.array([not dropped[t, j] for t, j in q], bool)
        assert kept.sum() == min(C, len(q))
        if kept.any() and (~kept).any():
            assert g[kept].min() >= g[~kept].max()
            # at equal gates the earlier entry is the kept one
            gmin = g[kept].min()
            if (g[~kept] == gmin).any():
                assert np.nonzero(kept & (g == gmin))[0].max() < np.nonzero(~kept & (g == gmin))[0].min()
        np.testing.assert_array_equal([slot[t, j] for (t, j), kk in zip(q, kept) if kk], np.arange(kept.sum()))
        np.testing.assert_array_equal([slot[t, j] for (t, j), kk in zip(q, kept) if not kk],
                                      C + np.arange((~kept).sum()))
