"""Seeded synthetic inputs for the token-choice MoE forward pass.

This module is shared by the CPU oracle, the tests and the benchmark, and by
nothing else.  It builds input tensors only: it holds none of the layer's
arithmetic (no logits, no routing, no expert maths).

Recipe (every tensor is reproducible from the workload's seed):

* numpy ``PCG64`` streams derived from ``SeedSequence(seed)``.  The root spawns
  one child per tensor role, in a fixed order (x, router weight, selection
  bias, row picks, routed experts, shared experts); big tensors are drawn in
  blocks of ``BLOCK`` elements, each block from its own grandchild stream, so
  the draw parallelises over threads and stays bit-identical.
* Normal draws are float32 ``standard_normal`` values multiplied by the
  float32 standard deviation ``1/sqrt(fan_in)`` (the "N(0, 1/fan_in)" of the
  workload descriptions is read as a variance).
* bf16 tensors are rounded from those float32 values with round-to-nearest-
  even and handed out as their raw 16-bit patterns (``np.uint16``).  The
  router weight is always float32.  Expert biases are zero.
* Weight layout is ``[experts, out_features, in_features]`` (row = output
  feature, contiguous over the input feature).

The five named workloads follow the sizes of the layer studied in the pages:
a tiny float32 layer, a Switch-style top-1 layer with two favoured experts, a
Mixtral-shaped SwiGLU layer, a DeepSeekMoE fine-grained layer with shared
experts, and a sigmoid-scored DeepSeek-V3-style stress layer with extreme and
duplicated token rows.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np

BLOCK = 1 << 22          # elements per independently seeded block
_THREADS = max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    d: int                 # model width
    E: int                 # routed experts
    k: int                 # experts per token
    d_ff: int              # routed expert hidden width
    act: str               # 'gelu' (2-matrix MLP) | 'swiglu' (3-matrix)
    score: str             # 'softmax' | 'sigmoid'
    renormalize: int       # -1 auto (k>1), 0 raw, 1 renormalise
    cf: float              # capacity factor
    dtype: str             # 'f32' | 'bf16' (router is float32 regardless)
    seed: int
    n_shared: int = 0
    d_ff_shared: int = 0
    logit_bias: str = ''   # '' | 'first_two_plus2' | 'log_rank' | 'last_minus30'
    select_bias: bool = False
    extreme_frac: float = 0.0
    extreme_scale: float = 0.0
    dup_frac: float = 0.0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    'tiny_f32': Workload('tiny_f32', T=64, d=32, E=4, k=2, d_ff=64, act='gelu',
                         score='softmax', renormalize=-1, cf=1.25, dtype='f32', seed=0),
    'switch_top1_skewed': Workload('switch_top1_skewed', T=4096, d=1024, E=16, k=1,
                                   d_ff=4096, act='gelu', score='softmax', renormalize=-1,
                                   cf=1.0, dtype='bf16', seed=1,
                                   logit_bias='first_two_plus2'),
    'mixtral_8x_top2': Workload('mixtral_8x_top2', T=8192, d=4096, E=8, k=2, d_ff=14336,
                                act='swiglu', score='softmax', renormalize=-1, cf=1.25,
                                dtype='bf16', seed=2),
    'deepseekmoe_fine': Workload('deepseekmoe_fine', T=16384, d=1024, E=64, k=6, d_ff=512,
                                 act='gelu', score='softmax', renormalize=-1, cf=1.25,
                                 dtype='bf16', seed=3, n_shared=2, d_ff_shared=512,
                                 logit_bias='log_rank'),
    'sigmoid_stress': Workload('sigmoid_stress', T=65536, d=2048, E=128, k=8, d_ff=1408,
                               act='swiglu', score='sigmoid', renormalize=1, cf=1.0,
                               dtype='bf16', seed=4, select_bias=True,
                               extreme_frac=0.01, extreme_scale=400.0, dup_frac=0.05),
}

# child-stream roles, in spawn order
_ROLES = ('x', 'w_router', 'select_bias', 'rows', 'experts', 'shared', 'extra')


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)

    def work(lo_hi):
        lo, hi = lo_hi
        v = flat_u[lo:hi].astype(np.uint32)
        lsb = (v >> 16) & 1
        v += 0x7FFF
        v += lsb
        v >>= 16
        flat_o[lo:hi] = v
    _blocks(flat_u.size, work)
    return out


def f32_of_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Any stored input tensor (float32 or bf16 bits) as float32 values."""
    return f32_of_bits(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def _blocks(n, fn):
    spans = [(i, min(n, i + BLOCK)) for i in range(0, n, BLOCK)]
    if len(spans) <= 1:
        for s in spans:
            fn(s)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, spans))


def _normal(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    """float32 N(0, std^2) tensor drawn in independently seeded blocks."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nblk = max(1, -(-n // BLOCK))
    kids = seq.spawn(nblk)
    s32 = np.float32(std)

    def work(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        seg = out[lo:hi]
        g.standard_normal(out=seg, dtype=np.float32)
        if s32 != np.float32(1.0):
            np.multiply(seg, s32, out=seg)
    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a32) if dtype == 'bf16' else a32


def _roots(w: Workload):
    return dict(zip(_ROLES, np.random.SeedSequence(w.seed).spawn(len(_ROLES))))


def router_inputs(w: Workload) -> dict:
    """x [T,d], w_router [d,E] f32, logit_bias [E]|None, select_bias [E]|None,
    plus the chosen extreme / duplicate row sets (for documentation and tests)."""
    r = _roots(w)
    x = _normal(r['x'], (w.T, w.d), 1.0)
    extreme = np.zeros(0, np.int64)
    dup_rows = np.zeros(0, np.int64)
    dup_src = np.zeros(0, np.int64)
    if w.extreme_frac > 0 or w.dup_frac > 0:
        g = np.random.Generator(np.random.PCG64(r['rows']))
        n_ext = int(round(w.extreme_frac * w.T))
        n_dup = int(round(w.dup_frac * w.T))
        perm = g.permutation(w.T)
        extreme = np.sort(perm[:n_ext])
        # duplicates never use row 0 (it has no lower-index source)
        rest = perm[n_ext:]
        rest = rest[rest > 0]
        dup_rows = np.sort(rest[:n_dup])
        if n_ext:
            x[extreme] *= np.float32(w.extreme_scale)
        if n_dup:
            dup_src = (g.random(n_dup) * dup_rows).astype(np.int64)   # uniform in [0, row)
            for r_, s_ in zip(dup_rows, dup_src):
                x[r_] = x[s_]
    xs = _store(x, w.dtype)
    w_router = _normal(r['w_router'], (w.d, w.E), 1.0 / math.sqrt(w.d))
    logit_bias = None
    if w.logit_bias == 'first_two_plus2':
        logit_bias = np.zeros(w.E, np.float32)
        logit_bias[:2] = 2.0
    elif w.logit_bias == 'log_rank':
        logit_bias = (-0.5 * np.log1p(np.arange(w.E, dtype=np.float64))).astype(np.float32)
    elif w.logit_bias == 'last_minus30':
        # the last expert is never chosen (an expert without rows)
        logit_bias = np.zeros(w.E, np.float32)
        logit_bias[-1] = -30.0
    select_bias = None
    if w.select_bias:
        g = np.random.Generator(np.random.PCG64(r['select_bias']))
        select_bias = g.uniform(-0.1, 0.1, w.E).astype(np.float32)
    return dict(x=xs, w_router=w_router, logit_bias=logit_bias, select_bias=select_bias,
                extreme_rows=extreme, dup_rows=dup_rows, dup_src=dup_src)


def expert_weights(w: Workload, e: int, shared: bool = False) -> dict:
    """Weights of routed expert e (or shared expert e): float32 or bf16 bits.

    GELU:   w_in [F,d], b_in [F], w_out [d,F], b_out [d]   (biases zero)
    SwiGLU: w_gate [F,d], w_up [F,d], w_out [d,F]          (no biases)
    Shared experts are always GELU MLPs of width d_ff_shared.
    """
    r = _roots(w)
    n = w.n_shared if shared else w.E
    if not 0 <= e < n:
        raise IndexError(e)
    seq = (r['shared'] if shared else r['experts']).spawn(n)[e]
    F = w.d_ff_shared if shared else w.d_ff
    act = 'gelu' if shared else w.act
    kids = seq.spawn(3)
    out = {}
    if act == 'gelu':
        out['w_in'] = _store(_normal(kids[0], (F, w.d), 1.0 / math.sqrt(w.d)), w.dtype)
        out['b_in'] = np.zeros(F, np.float32)
        out['w_out'] = _store(_normal(kids[2], (w.d, F), 1.0 / math.sqrt(F)), w.dtype)
        out['b_out'] = np.zeros(w.d, np.float32)
    else:
        out['w_gate'] = _store(_normal(kids[0], (F, w.d), 1.0 / math.sqrt(w.d)), w.dtype)
        out['w_up'] = _store(_normal(kids[1], (F, w.d), 1.0 / math.sqrt(w.d)), w.dtype)
        out['w_out'] = _store(_normal(kids[2], (w.d, F), 1.0 / math.sqrt(F)), w.dtype)
    return out


def all_expert_weights(w: Workload, shared: bool = False) -> dict:
    """Stacked [n, ...] weights of every routed (or shared) expert."""
    n = w.n_shared if shared else w.E
    per = [expert_weights(w, e, shared) for e in range(n)]
    return {key: np.stack([p[key] for p in per]) for key in per[0]} if per else {}


def random_logits(T: int, E: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """float32 logits ~ N(0, scale^2), for router-only cases fed with given logits."""
    return _normal(np.random.SeedSequence([seed, 0x10617]), (T, E), scale)


def random_indices(T: int, E: int, k: int, seed: int, skew: float = 0.0) -> np.ndarray:
    """[T,k] int32 distinct expert ids per token, best first; skew>0 favours low ids."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x1D5])))
    wts = np.exp(-skew * np.arange(E))
    wts = wts / wts.sum()
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = g.choice(E, size=k, replace=False, p=wts)
    return out


def tiny(name: str, **kw) -> Workload:
    """A small variant of a named workload (for tests on CPU or quick GPU checks)."""
    return WORKLOADS[name].with_(name=name + '_small', **kw)


def to_torch(a, device='cuda'):
    """A stored input tensor as a torch tensor on `device`: bf16 bit patterns
    become torch.bfloat16 (same bits), float32 stays float32."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)
