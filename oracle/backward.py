"""Backward pass of the token-choice MoE layer: the chain rule of the forward
definition in ``oracle.moe``, written out in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The training objective is  L = <dy, y> + alpha_aux * L_aux + alpha_z * L_z,
dy being the gradient arriving from above.  Sources: "Lab 18 -- Mixture of
experts" s.2 (the balance loss: f_i counts hard choices and carries no
gradient, the signal reaches the router through P_i; the router z-loss) and
its gate-value discussion in s.1 (with k = 1 and raw gates the gate is the
probability itself, which is how the router learns from the main loss);
"Lab 01" "The traps" (f is not differentiable); "Mixture of experts" lecture,
training a router.

Readings (listed in the design notes too):
  B1 the float32 rounding of the logits and the storage roundings of h, o
     and y are taken as the identity in the backward pass; every value the
     chain rule needs (h, o) is the stored (rounded) forward value, every
     value it can recompute (pre-activations) is recomputed in float64;
  B2 a dropped assignment contributes nothing to y, so its gate gets no
     gradient; top-k selection and capacity are piecewise constant and
     contribute none either;
  B3 the selection bias has no gradient (it enters the selection only);
  B4 a token that fell back to y = x passes dy straight to dx.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from synth import as_f32

from .moe import F64, expert_ffn, gelu, log_sigmoid, round_store, silu, softmax

SQRT_2PI = np.sqrt(2.0 * np.pi)


def gelu_grad(u):
    """d/du of u/2 (1 + erf(u/sqrt 2)) = Phi(u) + u phi(u), Phi and phi the
    standard normal distribution and density."""
    u = np.asarray(u, F64)
    return 0.5 * (1.0 + erf(u / np.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / SQRT_2PI


def silu_grad(u):
    """d/du of u sigma(u) = sigma(u) (1 + u (1 - sigma(u)))."""
    u = np.asarray(u, F64)
    s = np.exp(log_sigmoid(u))
    return s * (1.0 + u * (1.0 - s))


def expert_ffn_backward(a, wts, act, dtype, d_out):
    """Gradients of one expert MLP for rows a and output gradient d_out:
    (da, dict of weight gradients).  The hidden activation h the backward
    uses is the stored (rounded) one, as in the forward pass."""
    a = np.asarray(a, F64)
    d_out = np.asarray(d_out, F64)
    w_out = np.asarray(wts['w_out'], F64)
    if act == 'gelu':
        w_in = np.asarray(wts['w_in'], F64)
        u = a @ w_in.T
        if wts.get('b_in') is not None:
            u = u + np.asarray(wts['b_in'], F64)
        h = round_store(gelu(u), dtype)
        dh = d_out @ w_out
        du = dh * gelu_grad(u)
        g = {'w_out': d_out.T @ h, 'b_out': d_out.sum(axis=0), 'w_in': du.T @ a, 'b_in': du.sum(axis=0)}
        return du @ w_in, g
    if act == 'swiglu':
        w_gate = np.asarray(wts['w_gate'], F64)
        w_up = np.asarray(wts['w_up'], F64)
        gp = a @ w_gate.T
        up = a @ w_up.T
        h = round_store(silu(gp) * up, dtype)
        dh = d_out @ w_out
        d_up = dh * silu(gp)
        d_gp = dh * up * silu_grad(gp)
        g = {'w_out': d_out.T @ h, 'w_gate': d_gp.T @ a, 'w_up': d_up.T @ a}
        return d_gp @ w_gate + d_up @ w_up, g
    raise ValueError(act)


def router_backward(z, idx, dgates, score='softmax', renormalize=-1, f=None, alpha_aux=0.0, alpha_z=0.0,
                    n_tokens=None):
    """d L / d z for the logits z [T,E] (float64 values), given the gradient of
    the k gates of every token (0 for dropped ones), plus the balance and
    z-loss terms.

    Gates (see ``oracle.moe.gates``): renormalised softmax g = softmax(z_sel);
    raw softmax g = p_sel with p = softmax(z); normalised sigmoid
    g = softmax(log sigma(z_sel)); raw sigmoid g = sigma(z_sel).
    Balance loss: dL_aux/dp_ti = E f_i / T, through p = softmax(z) (or the
    normalised sigmoid scores softmax(log sigma(z))).  z-loss:
    dL_z/dz_ti = 2 LSE_t softmax(z)_ti / T.  ``n_tokens`` is the batch size T
    when z holds only some of the batch's rows (both losses are batch means).
    """
    z = np.asarray(z, F64)
    idx = np.asarray(idx)
    dg = np.asarray(dgates, F64)
    rows, E = z.shape
    T = rows if n_tokens is None else int(n_tokens)
    k = idx.shape[1]
    ren = (k > 1) if renormalize < 0 else bool(renormalize)
    dz = np.zeros((rows, E), F64)
    zs = np.take_along_axis(z, idx, axis=1)
    if score == 'softmax':
        if ren:
            g = softmax(zs)
            dzs = g * (dg - (g * dg).sum(axis=1, keepdims=True))
            np.put_along_axis(dz, idx, dzs, axis=1)
        else:
            p = softmax(z)
            dp = np.zeros((rows, E), F64)
            np.put_along_axis(dp, idx, dg, axis=1)
            dz += p * (dp - (p * dp).sum(axis=1, keepdims=True))
    elif score == 'sigmoid':
        sig = np.exp(log_sigmoid(zs))
        if ren:
            g = softmax(log_sigmoid(zs))
            dls = g * (dg - (g * dg).sum(axis=1, keepdims=True))     # through softmax of log sigma
            dzs = dls * (1.0 - sig)                                  # d log sigma(z)/dz = 1 - sigma(z)
        else:
            dzs = dg * sig * (1.0 - sig)
        np.put_along_axis(dz, idx, dzs, axis=1)
    else:
        raise ValueError(score)
    if alpha_aux and f is not None:
        v = alpha_aux * E * np.asarray(f, F64) / T                   # dL/dp_ti, the same for every t
        if score == 'softmax':
            p = softmax(z)
            dz += p * (v[None, :] - (p * v[None, :]).sum(axis=1, keepdims=True))
        else:
            q = softmax(log_sigmoid(z))
            dls = q * (v[None, :] - (q * v[None, :]).sum(axis=1, keepdims=True))
            dz += dls * (1.0 - np.exp(log_sigmoid(z)))
    if alpha_z:
        m = z.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
        dz += alpha_z * 2.0 * lse[:, None] * softmax(z) / T
    return dz


def probs_backward(z, dp, score='softmax'):
    """d/dz of <dp, p> for the full router probabilities p (softmax, or the
    sigmoid scores normalised over all experts, softmax of log sigma(z))."""
    z = np.asarray(z, F64)
    dp = np.asarray(dp, F64)
    if score == 'softmax':
        p = softmax(z)
        return p * (dp - (p * dp).sum(axis=1, keepdims=True))
    q = softmax(log_sigmoid(z))
    dls = q * (dp - (q * dp).sum(axis=1, keepdims=True))
    return dls * np.exp(log_sigmoid(-z))                             # d log sigma(z)/dz = sigma(-z)


def moe_backward_expert_choice(w, inp, experts, shared_experts, fwd, dy, alpha_aux=0.0, alpha_z=0.0,
                               dropped_output='residual', exact=False):
    """Gradients under expert-choice routing (``oracle.moe.expert_choice``):
    y_t = sum over the experts e that picked t of p_te FFN_e(x_t); the gate
    is the router probability itself, so the gate gradient of a pick lands on
    p_te and reaches z through the probabilities' Jacobian.  The picks are
    piecewise constant (no gradient); f_i = count_i / sum of counts.
    Returns the same keys as ``moe_backward``, with dgates replaced by
    dprobs [T,E] (the gradient of each picked probability, 0 elsewhere)."""
    T, E, d = w.T, w.E, w.d
    assert fwd['rows'].size == T, 'the backward pass needs the forward over every token'
    dy = np.asarray(dy, F64)
    x = np.asarray(inp['x'], F64) if exact else as_f32(inp['x']).astype(F64)
    cast = (lambda wts: {kk: (None if v is None else np.asarray(v, F64)) for kk, v in wts.items()}) if exact \
        else (lambda wts: {kk: (None if v is None else as_f32(v).astype(F64)) for kk, v in wts.items()})
    get = experts if callable(experts) else (lambda e: {kk: v[e] for kk, v in experts.items()})
    p = np.asarray(fwd['probs'], F64)
    sel = fwd['sel']
    dx = np.zeros((T, d), F64)
    dp = np.zeros((T, E), F64)
    grads = []
    for e in range(E):
        wts = cast(get(e))
        t_e = np.nonzero(sel[:, e] >= 0)[0]
        if t_e.size == 0:
            grads.append({kk: np.zeros_like(np.asarray(v, F64)) for kk, v in wts.items() if v is not None})
            continue
        a = x[t_e]
        _, o = expert_ffn(a, wts, w.act, w.dtype)
        dp[t_e, e] = (dy[t_e] * o).sum(axis=1)
        da, ge = expert_ffn_backward(a, wts, w.act, w.dtype, p[t_e, e][:, None] * dy[t_e])
        np.add.at(dx, t_e, da)
        if w.act == 'swiglu':
            ge = {kk: ge[kk] for kk in ('w_gate', 'w_up', 'w_out')}
        else:
            ge = {kk: ge[kk] if wts.get(kk) is not None else None for kk in ('w_in', 'b_in', 'w_out', 'b_out')}
        grads.append(ge)
    sgrads = []
    if shared_experts is not None and getattr(w, 'n_shared', 0) > 0:
        gs = shared_experts if callable(shared_experts) else \
            (lambda s: {kk: v[s] for kk, v in shared_experts.items()})
        for s_ in range(w.n_shared):
            da, ge = expert_ffn_backward(x, cast(gs(s_)), 'gelu', w.dtype, dy)
            dx += da
            sgrads.append(ge)
    elif dropped_output == 'residual':
        fb = ~(sel >= 0).any(axis=1)
        dx[fb] += dy[fb]
    z = np.asarray(fwd['logits'], F64)
    counts = (sel >= 0).sum(axis=0).astype(F64)
    v = np.zeros(E, F64)
    if alpha_aux:
        v = alpha_aux * E * (counts / max(1.0, counts.sum())) / T            # dL_aux/dp_ti
    dz = probs_backward(z, dp + v[None, :], w.score)
    if alpha_z:
        m = z.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
        dz += alpha_z * 2.0 * lse[:, None] * softmax(z) / T
    wr = np.asarray(inp['w_router'], F64)
    dx += dz @ wr.T
    return dict(dx=dx, dw_router=x.T @ dz, dlogit_bias=dz.sum(axis=0), dprobs=dp, dz=dz, experts=grads,
                shared=sgrads)


def moe_backward(w, inp, experts, shared_experts, fwd, dy, alpha_aux=0.0, alpha_z=0.0,
                 dropped_output='residual', exact=False):
    """Gradients of L = <dy, y> + alpha_aux L_aux + alpha_z L_z for the layer
    whose forward pass ``fwd`` (``oracle.moe.moe_forward`` over every token,
    same arguments) computed.

    Returns dx [T,d], dw_router [d,E], dlogit_bias [E], dgates [T,k],
    dz [T,E], experts: list of per-expert dicts (w_in, b_in, w_out, b_out for
    GELU; w_gate, w_up, w_out for SwiGLU), shared: list of per-shared-expert
    dicts.  The routed-expert step loops over experts, as the forward does.
    """
    T, E, k, d = w.T, w.E, w.k, w.d
    assert fwd['rows'].size == T, 'the backward pass needs the forward over every token'
    dy = np.asarray(dy, F64)
    x = np.asarray(inp['x'], F64) if exact else as_f32(inp['x']).astype(F64)
    cast = (lambda wts: {kk: (None if v is None else np.asarray(v, F64)) for kk, v in wts.items()}) if exact \
        else (lambda wts: {kk: (None if v is None else as_f32(v).astype(F64)) for kk, v in wts.items()})
    get = experts if callable(experts) else (lambda e: {kk: v[e] for kk, v in experts.items()})
    idx, g, dropped = fwd['idx'], fwd['gates'], fwd['dropped']
    kept = ~dropped
    dx = np.zeros((T, d), F64)
    dg = np.zeros((T, k), F64)
    grads = []
    for e in range(E):
        wts = cast(get(e))
        t_e, j_e = np.nonzero((idx == e) & kept)
        if t_e.size == 0:
            zero = {kk: np.zeros_like(np.asarray(v, F64)) for kk, v in wts.items() if v is not None}
            grads.append(zero)
            continue
        a = x[t_e]
        _, o = expert_ffn(a, wts, w.act, w.dtype)                   # the stored expert output
        dg[t_e, j_e] = (dy[t_e] * o).sum(axis=1)
        da, ge = expert_ffn_backward(a, wts, w.act, w.dtype, g[t_e, j_e][:, None] * dy[t_e])
        np.add.at(dx, t_e, da)
        if w.act == 'swiglu':
            ge = {kk: ge[kk] for kk in ('w_gate', 'w_up', 'w_out')}
        else:
            ge = {kk: ge[kk] if wts.get(kk) is not None else None for kk in ('w_in', 'b_in', 'w_out', 'b_out')}
        grads.append(ge)
    sgrads = []
    if shared_experts is not None and getattr(w, 'n_shared', 0) > 0:
        gs = shared_experts if callable(shared_experts) else \
            (lambda s: {kk: v[s] for kk, v in shared_experts.items()})
        for s_ in range(w.n_shared):
            da, ge = expert_ffn_backward(x, cast(gs(s_)), 'gelu', w.dtype, dy)
            dx += da
            sgrads.append(ge)
    elif dropped_output == 'residual':
        fb = ~kept.any(axis=1)
        dx[fb] += dy[fb]
    counts = np.bincount(np.asarray(idx).reshape(-1), minlength=E).astype(F64)
    f = counts / (T * k)
    dz = router_backward(fwd['logits'], idx, dg, w.score, w.renormalize, f, alpha_aux, alpha_z)
    wr = np.asarray(inp['w_router'], F64)
    dx += dz @ wr.T
    return dict(dx=dx, dw_router=x.T @ dz, dlogit_bias=dz.sum(axis=0), dgates=dg, dz=dz, experts=grads,
                shared=sgrads)
