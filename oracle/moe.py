"""Token-choice MoE forward pass: the plain definition, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (page titles, then section):
  [P1] "Phase 02 -- Mixture of Experts From Scratch" (concept map, takeaways)
  [P2] "Mixture of Experts -- parameters without the FLOPs" (s.2 the router,
       s.3 capacity)
  [P3] "Lab 18 -- Mixture of experts" (s.1 the layer and gate values, parameter
       table; s.2 load balancing; s.3 capacity and dropped tokens; "What to
       implement"; "Tips"; "Common bugs")
  [P4] "Lab 01 -- Router, Load Balancing, Capacity & the MoE Layer"
       ("Where to start", "The traps")
  [P5] "Mixture of experts" lecture field map (routing families; training a
       router; where the systems bill comes due; stability; DeepSeek V3)

Every function is the definition written out with numpy; matmul, exp, erf,
log1p and a stable lexicographic sort are the only library steps.  Inputs are
the exact values the device sees (bf16 tensors widened), logits are rounded to
float32 once, and stored intermediate tensors (expert hidden activations,
expert outputs, the layer output) are rounded to the layer's storage type at
the points listed in ``moe_forward``.

Readings taken where the pages are silent or disagree (each also listed in the
design notes):
  R1 capacity priority: rank-major (all first choices, then second choices;
     token order inside a rank) by default [P3 s.3, Tips, Common bugs];
     token-major is the alternative ordering [P4 "Where to start"].
  R2 a token whose every assignment drops and that has no shared expert
     outputs its input unchanged (residual pass-through) [P4 "Where to
     start"; P3 s.3]; ``dropped_output='zero'`` gives 0 instead.
  R3 f_i counts the T*k routed assignments before capacity [P3 s.2, "What to
     implement"; P4 "The traps"].
  R4 C = ceil(cf*T*k/E) evaluated in IEEE double in that order [P3 s.3];
     cf < 1 is an error [P4 "The traps"].
  R5 selection is on the logits (plus any selection bias) for softmax scores:
     top-k of the exact softmax is top-k of the logits [P3 "What to
     implement"; P2 s.2]; for sigmoid scores the key is
     fp32(sigmoid_spec(z)) + b in float32.
  R6 order: key descending, ties to the lower expert index, -0 == +0
     [P4 "The traps"]; this also reproduces P3's 0.92 example.
  R7 renormalise iff k > 1 unless told otherwise [P3 s.1 gate values].
  R8 a partially dropped token keeps its surviving gate unrenormalised
     [P3 s.3, Common bugs].
  R9 sigmoid gates and sigmoid P_i use the log domain so that saturated
     scores give no 0/0 [P3 s.1, DeepSeek-V3 note].
  R10 logit_bias enters the logits (hence p, gates, L_z); select_bias enters
     only the selection key [P3 s.2 auxiliary-loss-free balancing; P5].
  R11 exact-erf GELU; SwiGLU = SiLU(x W_gate^T) * (x W_up^T), no biases.
  R12 rounding points: logits -> float32; expert hidden h and expert output o
     -> storage type; y accumulated in float64 and rounded once.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from synth import as_f32

from .fp32spec import sigmoid_spec

F64 = np.float64


# ----------------------------------------------------------------------------- rounding
def round_bf16(v):
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits and float32's exponent range; the spacing at
    |v| in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below the normal range.
    Values past the largest finite bf16 become infinities.
    """
    v = np.asarray(v, dtype=F64)
    _, ex = np.frexp(v)
    ulp = np.ldexp(1.0, np.maximum(ex - 8, -133))
    r = np.rint(v / ulp) * ulp
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, v), r)
    return np.where(v == 0, v, r)


def round_store(v, dtype: str):
    """Round to the layer's storage type ('f32' or 'bf16'), returned as float64.
    'f64' stores exactly (the smooth layer that finite differences need)."""
    if dtype == 'f64':
        return np.asarray(v, dtype=F64)
    if dtype == 'f32':
        return np.asarray(v, dtype=F64).astype(np.float32).astype(F64)
    if dtype == 'bf16':
        return round_bf16(v)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- router
def router_logits(x, w_router, logit_bias=None):
    """z = x W_r (+ b), summed in float64 and rounded once to float32.

    [P3 s.1 layer equation; P2 s.2 router pseudo-code; P5 stability: the
    router runs in float32 whatever the ambient precision.]
    """
    z = np.asarray(x, F64) @ np.asarray(w_router, F64)
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, F64)[None, :]
    return z.astype(np.float32)


def selection_keys(z32, score='softmax', select_bias=None):
    """float32 keys the top-k ranks (R5, R10)."""
    z32 = np.asarray(z32, np.float32)
    if not np.all(np.isfinite(z32)):
        raise ValueError('router logits must be finite')
    key = sigmoid_spec(z32) if score == 'sigmoid' else z32.copy()
    if select_bias is not None:
        key = (key + np.asarray(select_bias, np.float32)[None, :]).astype(np.float32)
    return key + np.float32(0.0)          # -0 -> +0


def top_k(key, k):
    """Indices of the k largest keys per row, best first, ties to the lower index.

    A stable lexicographic sort on (-key, index) [P4 "The traps"; P3 "What
    to implement": experts best first].
    """
    key = np.asarray(key, np.float32)
    T, E = key.shape
    if not 1 <= k <= E:
        raise ValueError('need 1 <= k <= E')
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -key.astype(F64)), axis=-1)
    return order[:, :k].astype(np.int32)


def softmax(z):
    """Numerically stable softmax: subtract the row max [P4 "Where to start" 1]."""
    z = np.asarray(z, F64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def log_sigmoid(z):
    """log(sigmoid(z)) = -softplus(-z), stable for any magnitude."""
    z = np.asarray(z, F64)
    return np.where(z >= 0, -np.log1p(np.exp(-np.abs(z))), z - np.log1p(np.exp(-np.abs(z))))


def logsumexp(z):
    z = np.asarray(z, F64)
    m = z.max(axis=-1)
    return m + np.log(np.exp(z - m[..., None]).sum(axis=-1))


def probabilities(z32, score='softmax'):
    """Full-E router probabilities used for P_i.

    softmax: p = softmax(z)                       [P3 s.1, "What to implement"]
    sigmoid: q = s / sum(s), s = sigmoid(z), formed as softmax(log s)  (R9)
    """
    if score == 'sigmoid':
        return softmax(log_sigmoid(z32))
    return softmax(z32)


def gates(z32, idx, score='softmax', renormalize=-1):
    """Gate values of the selected experts, in selection order.

    softmax, renormalised: g_j = exp(z_j) / sum_{l in K} exp(z_l), which equals
      p_j / sum_K p  [P3 s.1 gate values; P2 s.2].
    softmax, raw (k == 1 default): g_j = p_j  [P3 s.1 gate values].
    sigmoid, normalised: g_j = s_j / sum_K s, in the log domain [P3 s.1
      DeepSeek-V3 note]; sigmoid, raw: g_j = s_j.
    The selection bias never enters a gate (R10).
    """
    z = np.asarray(z32, F64)
    idx = np.asarray(idx)
    k = idx.shape[1]
    ren = (k > 1) if renormalize < 0 else bool(renormalize)
    zs = np.take_along_axis(z, idx, axis=1)
    if score == 'sigmoid':
        return softmax(log_sigmoid(zs)) if ren else np.exp(log_sigmoid(zs))
    if ren:
        return softmax(zs)
    return np.take_along_axis(softmax(z), idx, axis=1)


def route(z32, k, score='softmax', renormalize=-1, select_bias=None):
    """(idx [T,k] int32, gates [T,k] f64, probs [T,E] f64) for given float32 logits."""
    key = selection_keys(z32, score, select_bias)
    idx = top_k(key, k)
    return idx, gates(z32, idx, score, renormalize), probabilities(z32, score)


# ----------------------------------------------------------------------------- losses
def load_balancing_loss(probs, idx, n_experts):
    """Switch auxiliary loss without its alpha: E * sum_i f_i P_i.

    f_i = (number of routed (token, slot) assignments to i) / (T k)   (R3)
    P_i = mean over tokens of the full router probability of i.
    [P3 s.2; P1 concept map; P4 "The traps": f divides by T*k.]
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=n_experts).astype(F64)
    f = counts / (T * k)
    P = np.asarray(probs, F64).mean(axis=0)
    return float(n_experts * np.sum(f * P))


def sequence_aux_loss(probs, idx, n_experts, seq_len):
    """Sequence-wise balance loss: the balance formula E * sum_i f_i P_i taken
    within each sequence of seq_len consecutive tokens (f over the sequence's
    seq_len*k routed choices, P the mean of its tokens' full router
    probabilities), averaged over the sequences.  ["Lab 18" s.2, the
    auxiliary-loss-free note: a small sequence-wise balance loss is kept;
    "Mixture of experts" lecture, DeepSeek section: the balancing unit is
    where the variants differ, with the same formula.]  No alpha.
    """
    idx = np.asarray(idx)
    probs = np.asarray(probs, F64)
    T, k = idx.shape
    if seq_len <= 0 or T % seq_len:
        raise ValueError('T must be a positive multiple of seq_len')
    n_seq = T // seq_len
    total = 0.0
    for b in range(n_seq):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        cnt = np.bincount(idx[rows].reshape(-1), minlength=n_experts).astype(F64)
        f = cnt / (seq_len * k)
        P = probs[rows].mean(axis=0)
        total += n_experts * float(np.sum(f * P))
    return total / n_seq


def update_select_bias(select_bias, counts, gamma, T, k):
    """Auxiliary-loss-free balancing: after a batch, lower the selection bias
    of every overloaded expert by gamma and raise it for every underloaded
    one; an expert exactly at the mean load T*k/E keeps its bias.  The load
    is the number of choices routed to the expert.  Each new bias is the
    float32 sum b_i +- gamma.  ["Lab 18" s.2 auxiliary-loss-free balancing
    (bias for selection only, a fixed small step) and its exercise 4 (step
    0.001); "Mixture of experts" lecture, DeepSeek section.]
    """
    b = np.asarray(select_bias, np.float32)
    counts = np.asarray(counts, np.int64)
    E = b.size
    # sign(mean - load), compared exactly as T*k versus load*E
    s = np.sign(T * k - counts * E).astype(F64)
    g = float(np.float32(gamma))
    return (b.astype(F64) + g * s).astype(np.float32)


def router_z_loss(z32):
    """(1/T) sum_t (log sum_i exp z_ti)^2  [P3 s.2 router z-loss; P1 concept map]."""
    lse = logsumexp(z32)
    return float(np.mean(lse * lse))


# ----------------------------------------------------------------------------- capacity
def capacity(T, k, E, cf, override=0):
    """C = ceil(cf * T * k / E) in IEEE double, or the given capacity (R4)."""
    if override and override > 0:
        return int(override)
    if not cf >= 1.0:
        raise ValueError('capacity_factor < 1 drops tokens even under perfect balance')
    return int(math.ceil(float(cf) * T * k / E))


def assign_capacity(idx, n_experts, C, priority='rank', scores=None):
    """Queue position of every assignment in its expert; dropped iff position >= C.

    Rank-major: walk rank j = 0..k-1, and inside a rank tokens in order
    [P3 s.3 GShard priority; Tips: flatten rank-major, one-hot, cumulative
    sum]. Token-major walks tokens, then ranks [P4 "Where to start" 4].
    'score': batch-prioritised routing, which ranks assignments by router
    score [P3 s.3, the V-MoE alternative]: in each expert the C assignments
    with the largest score (float32 ``scores`` [T,k], e.g. the gates; equal
    scores to the earlier one in the rank-major queue) are kept and numbered
    0.. in rank-major order; the dropped ones follow, numbered C.. in the
    same order.
    Returns slot [T,k] int32, dropped [T,k] bool, counts [E] int64,
    row_token [E,C] int32 (-1 where empty).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if priority == 'score':
        return _assign_by_score(idx, n_experts, C, np.asarray(scores, np.float32))
    cnt = [0] * n_experts
    slot = np.empty((T, k), np.int64)
    if priority == 'rank':
        order = ((t, j) for j in range(k) for t in range(T))
    elif priority == 'token':
        order = ((t, j) for t in range(T) for j in range(k))
    else:
        raise ValueError(priority)
    rows = idx.tolist()
    for t, j in order:
        e = rows[t][j]
        slot[t, j] = cnt[e]
        cnt[e] += 1
    dropped = slot >= C
    row_token = np.full((n_experts, C), -1, np.int32)
    keep = ~dropped
    row_token[idx[keep], slot[keep]] = np.nonzero(keep)[0]
    return slot.astype(np.int32), dropped, np.asarray(cnt, np.int64), row_token


def _assign_by_score(idx, n_experts, C, scores):
    T, k = idx.shape
    queue, _, counts, _ = assign_capacity(idx, n_experts, max(T, 1), 'rank')
    slot = np.empty((T, k), np.int64)
    dropped = np.zeros((T, k), bool)
    for e in range(n_experts):
        tt, jj = np.nonzero(idx == e)
        q = queue[tt, jj]
        order = np.argsort(q, kind='stable')             # this expert's rank-major queue
        tt, jj, q = tt[order], jj[order], q[order]
        sc = scores[tt, jj].astype(F64)
        best = np.lexsort((q, -sc))[:C]                  # score descending, queue position ascending
        keep = np.zeros(tt.size, bool)
        keep[best] = True
        slot[tt[keep], jj[keep]] = np.arange(int(keep.sum()))
        slot[tt[~keep], jj[~keep]] = C + np.arange(int((~keep).sum()))
        dropped[tt[~keep], jj[~keep]] = True
    row_token = np.full((n_experts, C), -1, np.int32)
    keep = ~dropped
    row_token[idx[keep], slot[keep]] = np.nonzero(keep)[0]
    return slot.astype(np.int32), dropped, counts, row_token


def dropless_rows(idx, n_experts, priority='rank'):
    """Dropless mode: every assignment is kept, and the experts' rows are laid
    back to back with no padding ["Lab 18" s.3, the alternatives to dropping:
    a capacity high enough that nothing is dropped, or block-sparse kernels
    without the limit; "Mixture of experts" lecture, systems section: ragged
    per-expert matmuls without padding].

    Row of (t, j) = (assignments routed to lower-numbered experts) + its
    queue position in its own expert, in the capacity queue's priority order.
    Returns row [T,k] int32, counts [E] int64, row_token [T*k] int32.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    # every expert receives at most T assignments, so a capacity of T drops none;
    # with nothing dropped, score priority numbers its rows in rank-major order
    pos, dropped, counts, _ = assign_capacity(idx, n_experts, max(T, 1),
                                              'rank' if priority == 'score' else priority)
    assert not dropped.any()
    first = np.concatenate([[0], np.cumsum(counts)[:-1]])
    row = (first[idx] + pos).astype(np.int32)
    row_token = np.empty(T * k, np.int32)
    row_token[row.ravel()] = np.repeat(np.arange(T, dtype=np.int32), k)
    return row, counts, row_token


def expert_choice(probs, C):
    """Expert-choice routing: every expert picks the C tokens with the largest
    router probability for it (all T tokens when T <= C), equal scores to the
    lower token index, and holds its picks in token order.  ["Lab 18"
    exercise 1 (each expert picks its top tokens: balance by construction, no
    dropping) and "Common extensions"; "Mixture of experts" lecture, routing
    families: the top of each expert's row of the token x expert score
    matrix.]  The scores are the given float32 probabilities (the decision is
    taken in the precision the router stores them in).
    Returns row_token [E, min(C, T)] int32 (ascending tokens) and sel [T, E]
    int32, the slot of token t in expert e or -1.
    """
    probs = np.asarray(probs, np.float32)
    T, E = probs.shape
    n = min(int(C), T)
    row_token = np.empty((E, n), np.int32)
    sel = np.full((T, E), -1, np.int32)
    tok = np.arange(T)
    for e in range(E):
        order = np.lexsort((tok, -probs[:, e].astype(F64)))     # score descending, token ascending
        picked = np.sort(order[:n])
        row_token[e] = picked
        sel[picked, e] = np.arange(n, dtype=np.int32)
    return row_token, sel


# ----------------------------------------------------------------------------- experts
def gelu(u):
    """Exact GELU: u/2 (1 + erf(u/sqrt 2))  (R11)."""
    u = np.asarray(u, F64)
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def silu(u):
    """SiLU(u) = u * sigmoid(u), with sigmoid(u) = (1 + tanh(u/2)) / 2 (no overflow)."""
    u = np.asarray(u, F64)
    return 0.5 * u * (1.0 + np.tanh(0.5 * u))


def expert_ffn(a, wts, act, dtype):
    """One expert on rows a [n,d]: (h rounded, o rounded).

    GELU: h = GELU(a W_in^T + b_in), o = h W_out^T + b_out  [P3 s.1: 2-matrix MLP]
    SwiGLU: h = SiLU(a W_gate^T) * (a W_up^T), o = h W_out^T  [P3 s.1: Mixtral's
    3-matrix expert; P5 expert geometry]
    """
    a = np.asarray(a, F64)
    if act == 'gelu':
        u = a @ np.asarray(wts['w_in'], F64).T
        if wts.get('b_in') is not None:
            u = u + np.asarray(wts['b_in'], F64)
        h = round_store(gelu(u), dtype)
        o = h @ np.asarray(wts['w_out'], F64).T
        if wts.get('b_out') is not None:
            o = o + np.asarray(wts['b_out'], F64)
    elif act == 'swiglu':
        g = a @ np.asarray(wts['w_gate'], F64).T
        u = a @ np.asarray(wts['w_up'], F64).T
        h = round_store(silu(g) * u, dtype)
        o = h @ np.asarray(wts['w_out'], F64).T
    else:
        raise ValueError(act)
    return h, round_store(o, dtype)


def combine(routed, shared=None, x=None, any_kept=None, dropped_output='residual'):
    """y_t = sum over kept (t,j) of g_tj o_tj  (+ S_t); fallback x_t.

    ``routed`` already holds the gate-weighted sum of every kept assignment
    (float64).  A token with no kept assignment and no shared expert takes its
    input unchanged (or 0 with ``dropped_output='zero'``).
    [P3 s.1 layer equation; P3 s.3: a dropped slot contributes nothing and a
    fully dropped token reaches the next layer unchanged; P4 "Where to start"
    5: the residual fallback; P1 concept map: shared expert for every token.]
    """
    y = np.array(routed, dtype=F64)
    if shared is not None:
        y += shared
    elif any_kept is not None:
        fb = ~np.asarray(any_kept)
        y[fb] = np.asarray(x, F64)[fb] if dropped_output == 'residual' else 0.0
    return y


# ----------------------------------------------------------------------------- forward
def moe_forward(w, inp, experts, shared_experts=None, rows=None, priority='rank',
                capacity_override=0, dropped_output='residual', logits=None, dropless=False,
                routing='token', exact=False):
    """The whole layer.

    w: a ``synth.Workload``-like object (T, d, E, k, act, score, renormalize,
       cf, dtype, n_shared).
    inp: dict with x (float32 values), w_router, logit_bias, select_bias.
    experts: callable e -> dict of expert e's weights (float32 values), or a
       dict of stacked arrays.
    shared_experts: same for the shared experts (or None).
    rows: optional sorted token ids; expert maths and y only for those rows
       (routing, capacity and losses always use every token).
    logits: optional given float32 logits (then x is used only for expert maths).
    dropless: keep every assignment (capacity T); 'slot' and 'row_token' are
       then the packed rows of ``dropless_rows``.
    routing: 'token' (token choice, the default) or 'expert' (expert choice:
       every expert takes its C best tokens by float32 probability, the gate
       is that probability).
    exact: no float32 rounding of x, the weights or the logits' values (the
       selection still ranks the float32 keys); with w.dtype 'f64' the layer
       is then smooth wherever no choice changes, as finite differences need.

    Steps: logits -> keys -> top-k -> gates/probs -> capacity -> experts ->
    combine, with the losses beside [P3 "What to implement" 1-5; P4 build
    order].
    """
    x = inp['x']
    T, E, k, d = w.T, w.E, w.k, w.d
    if exact:
        z = np.asarray(x, F64) @ np.asarray(inp['w_router'], F64)
        if inp.get('logit_bias') is not None:
            z = z + np.asarray(inp['logit_bias'], F64)[None, :]
    else:
        z = router_logits(as_f32(x), inp['w_router'], inp.get('logit_bias')) if logits is None \
            else np.asarray(logits, np.float32)
    idx, g, probs = route(z, k, w.score, w.renormalize, inp.get('select_bias'))
    lse = logsumexp(z)
    if routing == 'expert':
        return _expert_choice_forward(w, inp, experts, shared_experts, rows, capacity_override,
                                      dropped_output, z, idx, g, probs, lse, exact)
    if dropless:
        C = T
        slot, counts, row_token = dropless_rows(idx, E, priority)
        dropped = np.zeros((T, k), bool)
    else:
        C = capacity(T, k, E, w.cf, capacity_override)
        slot, dropped, counts, row_token = assign_capacity(idx, E, C, priority,
                                                           scores=np.asarray(g, np.float32))
    l_aux = load_balancing_loss(probs, idx, E)
    l_z = float(np.mean(lse * lse))

    rows = np.arange(T) if rows is None else np.asarray(rows)
    sel = np.zeros(T, bool)
    sel[rows] = True
    pos = np.full(T, -1, np.int64)
    pos[rows] = np.arange(rows.size)
    kept = ~dropped
    xa = np.asarray(x, F64) if exact else as_f32(x)
    wcast = (lambda wts: {kk: (None if v is None else np.asarray(v, F64)) for kk, v in wts.items()}) \
        if exact else _f32_weights
    get = experts if callable(experts) else (lambda e: {kk: v[e] for kk, v in experts.items()})
    routed = np.zeros((rows.size, d), F64)
    for e in range(E):
        # loop over experts, never over tokens [P3 Tips]; a token picks an
        # expert at most once, so t_e has no repeats
        t_e, j_e = np.nonzero((idx == e) & kept & sel[:, None])
        if t_e.size == 0:
            continue
        _, o = expert_ffn(xa[t_e].astype(F64), wcast(get(e)), w.act, w.dtype)
        routed[pos[t_e]] += g[t_e, j_e][:, None] * o

    S = None
    if shared_experts is not None and getattr(w, 'n_shared', 0) > 0:
        gs = shared_experts if callable(shared_experts) else \
            (lambda s: {kk: v[s] for kk, v in shared_experts.items()})
        S = np.zeros((rows.size, d), F64)
        for s in range(w.n_shared):
            _, o = expert_ffn(xa[rows].astype(F64), wcast(gs(s)), 'gelu', w.dtype)
            S += o
    any_kept = kept.any(axis=1)[rows]
    y = combine(routed, S, xa[rows], any_kept, dropped_output)
    y = round_store(y, w.dtype)

    kept_e = np.minimum(counts, C)
    n_kept = int(kept_e.sum())
    stats = dict(kept=n_kept, dropped=T * k - n_kept,
                 fallback=int((~kept.any(axis=1)).sum()) if S is None else 0,
                 pad=0 if dropless else E * C - n_kept)
    return dict(y=y, rows=rows, logits=z, idx=idx, gates=g, probs=probs, lse=lse,
                capacity=C, slot=slot, dropped=dropped, counts=counts,
                row_token=row_token, l_aux=l_aux, l_z=l_z, stats=stats)


def _expert_choice_forward(w, inp, experts, shared_experts, rows, capacity_override, dropped_output,
                           z, idx, g, probs, lse, exact=False):
    """The layer under expert-choice routing (see ``expert_choice``): y_t is
    the sum over the experts that picked t of p_te * FFN_e(x_t) (+ shared
    experts); a token no expert picked passes through (or 0) as under token
    choice.  f_i in the balance loss counts picks: count_i / (sum of counts)."""
    T, E, k, d = w.T, w.E, w.k, w.d
    C = capacity(T, k, E, w.cf, capacity_override)
    row_token, sel = expert_choice(np.asarray(probs, np.float32), C)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    sel_rows = np.zeros(T, bool)
    sel_rows[rows] = True
    pos = np.full(T, -1, np.int64)
    pos[rows] = np.arange(rows.size)
    xa = np.asarray(inp['x'], F64) if exact else as_f32(inp['x'])
    wcast = (lambda wts: {kk: (None if v is None else np.asarray(v, F64)) for kk, v in wts.items()}) \
        if exact else _f32_weights
    get = experts if callable(experts) else (lambda e: {kk: v[e] for kk, v in experts.items()})
    routed = np.zeros((rows.size, d), F64)
    for e in range(E):
        t_e = row_token[e][sel_rows[row_token[e]]]
        if t_e.size == 0:
            continue
        _, o = expert_ffn(xa[t_e].astype(F64), wcast(get(e)), w.act, w.dtype)
        routed[pos[t_e]] += probs[t_e, e][:, None] * o
    S = None
    if shared_experts is not None and getattr(w, 'n_shared', 0) > 0:
        gs = shared_experts if callable(shared_experts) else \
            (lambda s_: {kk: v[s_] for kk, v in shared_experts.items()})
        S = np.zeros((rows.size, d), F64)
        for s_ in range(w.n_shared):
            _, o = expert_ffn(xa[rows].astype(F64), wcast(gs(s_)), 'gelu', w.dtype)
            S += o
    picked = (sel >= 0).any(axis=1)
    y = round_store(combine(routed, S, xa[rows], picked[rows], dropped_output), w.dtype)
    counts = (sel >= 0).sum(axis=0).astype(np.int64)
    f = counts / max(1, counts.sum())
    l_aux = float(E * np.sum(f * np.asarray(probs, F64).mean(axis=0)))
    n_kept = int(counts.sum())
    stats = dict(kept=n_kept, dropped=0, fallback=int((~picked).sum()) if S is None else 0,
                 pad=E * C - n_kept)
    return dict(y=y, rows=rows, logits=z, idx=idx, gates=g, probs=probs, lse=lse, capacity=C,
                row_token=row_token, sel=sel, counts=counts, l_aux=l_aux,
                l_z=float(np.mean(lse * lse)), stats=stats)


def _f32_weights(wts):
    return {kk: (None if v is None else as_f32(v)) for kk, v in wts.items()}


# ----------------------------------------------------------------------------- accounting
def ffn_params(d, d_ff, act='gelu'):
    """Weights of one expert: 2 d d_ff (GELU MLP) or 3 d d_ff (SwiGLU) [P3 s.1]."""
    return (2 if act == 'gelu' else 3) * d * d_ff


def moe_param_counts(d, d_ff, n_experts, k, n_shared=0, d_ff_shared=None, act='gelu'):
    """(total, active) parameters of one MoE layer, router and shared experts
    included [P3 parameter table, "What to implement" 6; P1 takeaways]."""
    d_ff_shared = d_ff if d_ff_shared is None else d_ff_shared
    router = d * n_experts
    shared = n_shared * ffn_params(d, d_ff_shared, act)
    per = ffn_params(d, d_ff, act)
    return n_experts * per + router + shared, k * per + router + shared


def sparsity_ratio(d, d_ff, n_experts, k, n_shared=0, act='gelu'):
    """active / total parameters; exactly 1.0 when k == E [P4 "The traps"; P1]."""
    total, active = moe_param_counts(d, d_ff, n_experts, k, n_shared, act=act)
    return active / total
