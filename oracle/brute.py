"""Pure-Python per-token brute force for tiny MoE inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Written separately from ``oracle.moe`` (no shared helpers) so that the two can
check each other: logits are summed one product at a time, top-k is a
selection by repeated maximum, capacity slots are counted by scanning every
earlier assignment in priority order, and each token runs its experts as
explicit loops.  "Checked against a per-token reference" is how the Lab 18
page ("What to implement" 5) pins the layer; this is that reference.

Python floats are IEEE doubles.  float32 operations are emulated by rounding
the double result of each +, -, *, / of float32 operands back to float32,
which yields the correctly rounded float32 result for those operations.
"""
import math
import struct


def f32(v):
    return struct.unpack('<f', struct.pack('<f', v))[0]


def bf16(v):
    """Nearest bf16 (ties to even) of a double: round it to 8 significant bits
    (spacing 2^-133 below the normal range)."""
    if v == 0.0 or math.isinf(v) or math.isnan(v):
        return v
    m, e = math.frexp(v)               # v = m * 2^e, 0.5 <= |m| < 1
    scale = 2.0 ** max(e - 8, -133)
    q = v / scale
    r = round(q)                        # Python rounds half to even
    out = r * scale
    if abs(out) > (2.0 - 2.0 ** -7) * 2.0 ** 127:
        return math.copysign(math.inf, v)
    return out


def store(v, dtype):
    return f32(v) if dtype == 'f32' else bf16(v)


# float32 sigmoid selection key, emulated one float32 operation at a time
_INV_LN2 = f32(1.0 / math.log(2.0))
_LN2_HI = f32(0.693145751953125)
_LN2_LO = f32(math.log(2.0) - 0.693145751953125)
_C = [f32(1.0 / math.factorial(i)) for i in range(8)]


def _exp_key(a):
    if a > 88.0:
        return math.inf
    if a < -87.0:
        return 0.0
    t = f32(a * _INV_LN2)
    n = float(round(t))                 # half to even
    r = f32(f32(a - f32(n * _LN2_HI)) - f32(n * _LN2_LO))
    p = _C[7]
    for c in reversed(_C[:7]):
        p = f32(f32(p * r) + c)
    return f32(math.ldexp(p, int(n)))


def sigmoid_key(z):
    e = _exp_key(-z)
    return 0.0 if math.isinf(e) else f32(1.0 / f32(1.0 + e))


def forward(x, w_router, logit_bias, select_bias, experts, shared, *, k, act, score,
            renormalize, C, dtype, priority='rank', dropped_output='residual', routing='token'):
    """Per-token reference.  Lists of lists in, dict of lists out.

    x [T][d]; w_router [d][E]; experts[e] dict with lists (w_in [F][d], b_in,
    w_out [d][F], b_out) or (w_gate, w_up, w_out); shared: list of GELU expert
    dicts (may be empty).  routing='expert': each expert takes, by repeated
    maximum over the tokens, the C largest float32-rounded probabilities
    (equal -> lower token), and the gate is the probability itself.
    """
    T, d, E = len(x), len(x[0]), len(w_router[0])
    # logits, one product at a time, then one float32 rounding
    z = []
    for t in range(T):
        row = []
        for i in range(E):
            s = 0.0
            for c in range(d):
                s += x[t][c] * w_router[c][i]
            if logit_bias is not None:
                s += logit_bias[i]
            row.append(f32(s))
        z.append(row)
    # selection by repeated maximum: larger key wins, equal keys -> lower index
    idx, gate, probs, lse = [], [], [], []
    for t in range(T):
        keys = []
        for i in range(E):
            kv = sigmoid_key(z[t][i]) if score == 'sigmoid' else z[t][i]
            if select_bias is not None:
                kv = f32(kv + select_bias[i])
            keys.append(kv)
        chosen = []
        for _ in range(k):
            best = None
            for i in range(E):
                if i in chosen:
                    continue
                if best is None or keys[i] > keys[best]:
                    best = i
            chosen.append(best)
        idx.append(chosen)
        m = max(z[t])
        ssum = sum(math.exp(v - m) for v in z[t])
        lse.append(m + math.log(ssum))
        ren = (k > 1) if renormalize < 0 else bool(renormalize)
        if score == 'softmax':
            probs.append([math.exp(v - m) / ssum for v in z[t]])
            if ren:
                tot = sum(math.exp(z[t][i] - m) for i in chosen)
                gate.append([math.exp(z[t][i] - m) / tot for i in chosen])
            else:
                gate.append([probs[t][i] for i in chosen])
        else:
            def sig(v):
                return 1.0 / (1.0 + math.exp(-v)) if v > -700 else math.exp(v)
            sv = [sig(v) for v in z[t]]
            tot_all = sum(sv)
            probs.append([s_ / tot_all for s_ in sv])
            if ren:
                tot = sum(sv[i] for i in chosen)
                gate.append([sv[i] / tot for i in chosen])
            else:
                gate.append([sv[i] for i in chosen])
    if routing == 'expert':
        picks = []                       # picks[e] = tokens chosen by expert e, ascending
        for i in range(E):
            mine = []
            for _ in range(min(C, T)):
                best = None
                for t in range(T):
                    if t in mine:
                        continue
                    if best is None or f32(probs[t][i]) > f32(probs[best][i]):
                        best = t
                mine.append(best)
            picks.append(sorted(mine))
    # capacity: slot = number of earlier assignments (priority order) to the same expert
    seq = [(t, j) for t in range(T) for j in range(k)] if priority == 'token' else \
        [(t, j) for j in range(k) for t in range(T)]
    slot = [[0] * k for _ in range(T)]
    for p, (t, j) in enumerate(seq):
        e = idx[t][j]
        slot[t][j] = sum(1 for (t2, j2) in seq[:p] if idx[t2][j2] == e)
    if priority == 'score':
        # per expert: keep the C largest float32 gates by repeated maximum over
        # its queue (equal -> earlier in the queue); kept numbered first
        for e in range(E):
            queue = [(t, j) for (t, j) in seq if idx[t][j] == e]
            kept = []
            for _ in range(min(C, len(queue))):
                best = None
                for q in queue:
                    if q in kept:
                        continue
                    if best is None or f32(gate[q[0]][q[1]]) > f32(gate[best[0]][best[1]]):
                        best = q
                kept.append(best)
            nk = nd = 0
            for (t, j) in queue:
                if (t, j) in kept:
                    slot[t][j] = nk
                    nk += 1
                else:
                    slot[t][j] = C + nd
                    nd += 1
    dropped = [[slot[t][j] >= C for j in range(k)] for t in range(T)]

    def run(wts, a, kind):
        if kind == 'gelu':
            F = len(wts['w_in'])
            h = []
            for f in range(F):
                u = sum(wts['w_in'][f][c] * a[c] for c in range(d)) + wts['b_in'][f]
                h.append(store(0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))), dtype))
            return [store(sum(wts['w_out'][o][f] * h[f] for f in range(F)) + wts['b_out'][o],
                          dtype) for o in range(d)]
        F = len(wts['w_gate'])
        h = []
        for f in range(F):
            g = sum(wts['w_gate'][f][c] * a[c] for c in range(d))
            u = sum(wts['w_up'][f][c] * a[c] for c in range(d))
            h.append(store(g / (1.0 + math.exp(-g)) * u, dtype))
        return [store(sum(wts['w_out'][o][f] * h[f] for f in range(F)), dtype)
                for o in range(d)]

    y = []
    for t in range(T):
        acc = [0.0] * d
        any_kept = False
        mine = [(i, probs[t][i]) for i in range(E) if t in picks[i]] if routing == 'expert' else \
            [(idx[t][j], gate[t][j]) for j in range(k) if not dropped[t][j]]
        for i, gv in mine:
            any_kept = True
            out = run(experts[i], x[t], act)
            for c in range(d):
                acc[c] += gv * out[c]
        for s_ in shared:
            out = run(s_, x[t], 'gelu')
            for c in range(d):
                acc[c] += out[c]
        if not any_kept and not shared:
            acc = list(x[t]) if dropped_output == 'residual' else [0.0] * d
        y.append([store(v, dtype) for v in acc])
    if routing == 'expert':
        counts = [len(picks[e]) for e in range(E)]
        sel = [[picks[e].index(t) if t in picks[e] else -1 for e in range(E)] for t in range(T)]
    else:
        counts = [sum(1 for t in range(T) for j in range(k) if idx[t][j] == e) for e in range(E)]
        sel = None
    l_aux = E * sum((counts[i] / sum(counts)) * (sum(probs[t][i] for t in range(T)) / T)
                    for i in range(E))
    l_z = sum(v * v for v in lse) / T
    return dict(y=y, logits=z, idx=idx, gates=gate, probs=probs, lse=lse, slot=slot,
                dropped=dropped, counts=counts, l_aux=l_aux, l_z=l_z, sel=sel)
