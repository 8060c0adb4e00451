"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
calls through the C ABI, and the comparison rules.

Comparison rules (the bar the tests hold the HIP path to):
  * integer and index outputs (idx, slot, dropped, counts, row_token, sel,
    stats): bit-exact, given identical float32 logits (or probabilities);
  * float32 outputs: max-relative error ||a - b||_inf / ||b||_inf <= 1e-5;
  * bf16 layer output y: max-relative error <= 2e-2;
  * losses: |a - b| / |b| <= 1e-5;
  * end to end, the oracle runs twice: on its own logits, which the GPU's must
    match within the float32 dot-product error bound and which must give the
    same choices for every token that is not near a tie (an adjacent gap among
    its top-(k+1) keys below max(1e-5, what the observed logit difference can
    move a key)); and on the GPU's logits, against which every output is held
    to the bars above over all tokens.
"""
import os

import numpy as np
import torch

import synth
from oracle import moe as O

DEV = 'cuda'

# The errors the comparisons measured: per test (pytest's id of the running
# test) and quantity, the worst value seen.  conftest prints them as a table
# at the end of the session, so a drift towards a bar shows before it fails.
PARITY = {}


def record(quantity, err):
    test = os.environ.get('PYTEST_CURRENT_TEST', '?').split(' ')[0]
    row = PARITY.setdefault(test, {})
    row[quantity] = max(row.get(quantity, 0.0), float(err))


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
