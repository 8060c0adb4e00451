"""MI355X-native token-choice mixture-of-experts forward pass.

A thin ctypes binding over ``libmoe.so`` (hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/moe.h``).  Every step of the layer runs
in those kernels; this module only marshals arguments: torch supplies device
memory and the current stream.  The entry points keep the C names:

    moe_validate, moe_workspace_bytes, moe_route, moe_dispatch,
    moe_expert_ffn, moe_combine, moe_aux_losses, moe_forward

If the library is not built, importing this package raises ImportError; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, 'libmoe.so')

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_GELU, MOE_SWIGLU = 0, 1
MOE_RANK_MAJOR, MOE_TOKEN_MAJOR, MOE_SCORE_PRIORITY = 0, 1, 2
MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE = 0, 1

EXPORTS = ('moe_validate', 'moe_workspace_bytes', 'moe_route', 'moe_dispatch', 'moe_expert_ffn',
           'moe_combine', 'moe_aux_losses', 'moe_forward', 'moe_last_error')


class moe_config(ctypes.Structure):
    _fields_ = [('T', ctypes.c_int64), ('d', ctypes.c_int32), ('E', ctypes.c_int32),
                ('k', ctypes.c_int32), ('d_ff', ctypes.c_int32), ('n_shared', ctypes.c_int32),
                ('d_ff_shared', ctypes.c_int32), ('capacity_factor', ctypes.c_double),
                ('capacity_override', ctypes.c_int64), ('renormalize', ctypes.c_int32),
                ('score', ctypes.c_int32), ('act', ctypes.c_int32), ('dtype', ctypes.c_int32),
                ('priority', ctypes.c_int32), ('dropped_output', ctypes.c_int32),
                ('dropless', ctypes.c_int32), ('routing', ctypes.c_int32), ('save_preact', ctypes.c_int32)]


_P = ctypes.c_void_p


class moe_weights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ('w_router', 'logit_bias', 'select_bias', 'w_in', 'w_gate', 'b_in',
                                  'w_out', 'b_out', 'ws_in', 'bs_in', 'ws_out', 'bs_out')]


class moe_outputs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ('y', 'idx', 'gates', 'slot', 'dropped', 'counts', 'losses',
                                  'stats', 'logits', 'probs', 'lse', 'sel')]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, _P) for n in ('dx', 'dw_router', 'dlogit_bias', 'dw_in', 'dw_gate', 'db_in', 'dw_out', 'db_out',
                                  'dws_in', 'dbs_in', 'dws_out', 'dbs_out', 'dgates', 'dlogits')]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f'{LIB_PATH} is not built: run `python mixture_experts_layer_20_amd/build.py`')
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    cfgp = ctypes.POINTER(moe_config)
    sig = {
        'moe_validate': (st, [cfgp, ctypes.POINTER(ctypes.c_int64)]),
        'moe_workspace_bytes': (ctypes.c_size_t, [cfgp]),
        'moe_route': (st, [cfgp] + [_P] * 11),
        'moe_dispatch': (st, [cfgp] + [_P] * 9),
        'moe_dispatch_by_score': (st, [cfgp] + [_P] * 10),
        'moe_dispatch_noalloc': (st, [cfgp] + [_P] * 8),
        'moe_expert_ffn': (st, [cfgp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _P, _P, _P,
                                ctypes.c_int64, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
        'moe_expert_ffn_packed': (st, [cfgp, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P, _P,
                                       ctypes.c_int64, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
        'moe_sequence_aux_loss': (st, [cfgp, ctypes.c_int64, _P, _P, _P, _P, _P]),
        'moe_update_select_bias': (st, [cfgp, _P, _P, ctypes.c_float, _P]),
        'moe_combine': (st, [cfgp] + [_P] * 9),
        'moe_expert_choice': (st, [cfgp] + [_P] * 6),
        'moe_combine_expert_choice': (st, [cfgp] + [_P] * 7),
        'moe_aux_losses': (st, [cfgp, _P, _P, _P, _P, _P]),
        'moe_forward': (st, [cfgp, ctypes.POINTER(moe_weights), _P, ctypes.POINTER(moe_outputs),
                             _P, _P]),
        'moe_forward_events': (st, [cfgp, ctypes.POINTER(moe_weights), _P, ctypes.POINTER(moe_outputs),
                                    _P, _P, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
        'moe_backward_workspace_bytes': (ctypes.c_size_t, [cfgp]),
        'moe_backward': (st, [cfgp, ctypes.POINTER(moe_weights), _P, ctypes.POINTER(moe_outputs), _P, _P,
                              ctypes.c_float, ctypes.c_float, ctypes.POINTER(moe_grads), _P, _P]),
        'moe_last_error': (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

_ENUMS = {
    'score': {'softmax': MOE_SOFTMAX, 'sigmoid': MOE_SIGMOID},
    'act': {'gelu': MOE_GELU, 'swiglu': MOE_SWIGLU},
    'dtype': {'f32': MOE_F32, 'float32': MOE_F32, 'bf16': MOE_BF16, 'bfloat16': MOE_BF16},
    'priority': {'rank': MOE_RANK_MAJOR, 'token': MOE_TOKEN_MAJOR, 'score': MOE_SCORE_PRIORITY},
    'dropped_output': {'residual': 0, 'zero': 1},
    'routing': {'token': MOE_TOKEN_CHOICE, 'expert': MOE_EXPERT_CHOICE},
}


def _enum(kind, v):
    return _ENUMS[kind][v] if isinstance(v, str) else int(v)


def make_config(T, d, E, k, d_ff, *, n_shared=0, d_ff_shared=0, capacity_factor=1.25,
                capacity_override=0, renormalize=-1, score='softmax', act='gelu', dtype='bf16',
                priority='rank', dropped_output='residual', dropless=False,
                routing='token', save_preact=False) -> moe_config:
    return moe_config(T=T, d=d, E=E, k=k, d_ff=d_ff, n_shared=n_shared, d_ff_shared=d_ff_shared,
                      capacity_factor=float(capacity_factor), capacity_override=capacity_override,
                      renormalize=renormalize, score=_enum('score', score), act=_enum('act', act),
                      dtype=_enum('dtype', dtype), priority=_enum('priority', priority),
                      dropped_output=_enum('dropped_output', dropped_output), dropless=int(bool(dropless)),
                      routing=_enum('routing', routing), save_preact=int(bool(save_preact)))


def config_from_workload(w, **over) -> moe_config:
    """moe_config for a ``synth.Workload``-like object (keyword overrides allowed)."""
    kw = dict(n_shared=w.n_shared, d_ff_shared=w.d_ff_shared, capacity_factor=w.cf,
              renormalize=w.renormalize, score=w.score, act=w.act, dtype=w.dtype)
    kw.update(over)
    return make_config(w.T, w.d, w.E, w.k, w.d_ff, **kw)


def torch_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


class MoEError(RuntimeError):
    pass


def _check(status):
    if status == MOE_OK:
        return
    msg = _lib.moe_last_error().decode()
    if status == MOE_EINVAL:
        raise ValueError(msg)
    if status == MOE_EUNSUPPORTED:
        raise NotImplementedError(msg)
    raise MoEError(msg)


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f'{name} must be a torch.Tensor')
    if t.device.type != 'cuda':
        raise ValueError(f'{name} must be a device tensor')
    if not t.is_contiguous():
        raise ValueError(f'{name} must be contiguous')
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f'{name} must be {dtype}, got {t.dtype}')
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, 'cuda_stream') else int(stream)


# ----------------------------------------------------------------------------- host-only calls
def moe_validate(cfg: moe_config) -> int:
    """Capacity C of a valid configuration; ValueError otherwise."""
    cap = ctypes.c_int64(0)
    _check(_lib.moe_validate(ctypes.byref(cfg), ctypes.byref(cap)))
    return cap.value


def moe_workspace_bytes(cfg: moe_config) -> int:
    n = _lib.moe_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        moe_validate(cfg)
    return n


def workspace(cfg: moe_config, device='cuda') -> torch.Tensor:
    return torch.empty(max(1, moe_workspace_bytes(cfg)), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- device calls
def moe_route(cfg, x, w_router, logit_bias, select_bias, logits, probs, idx, gates, lse, ws,
              stream=None):
    dt = torch_dtype(cfg)
    _check(_lib.moe_route(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(w_router, 'w_router', torch.float32),
                          _ptr(logit_bias, 'logit_bias', torch.float32),
                          _ptr(select_bias, 'select_bias', torch.float32),
                          _ptr(logits, 'logits', torch.float32), _ptr(probs, 'probs', torch.float32),
                          _ptr(idx, 'idx', torch.int32), _ptr(gates, 'gates', torch.float32),
                          _ptr(lse, 'lse', torch.float32), _ptr(ws, 'ws'), _stream(stream)))


def moe_dispatch(cfg, x, idx, slot, dropped, counts, row_token, xe, ws, stream=None):
    dt = torch_dtype(cfg)
    _check(_lib.moe_dispatch(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(idx, 'idx', torch.int32),
                             _ptr(slot, 'slot', torch.int32), _ptr(dropped, 'dropped', torch.uint8),
                             _ptr(counts, 'counts', torch.int32),
                             _ptr(row_token, 'row_token', torch.int32), _ptr(xe, 'xe', dt),
                             _ptr(ws, 'ws'), _stream(stream)))


def moe_dispatch_noalloc(cfg, x, idx, slot, dropped, counts, row_token, xe, stream=None):
    """moe_dispatch with no workspace: the library's fixed per-GPU scratch."""
    dt = torch_dtype(cfg)
    _check(_lib.moe_dispatch_noalloc(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(idx, 'idx', torch.int32),
                                     _ptr(slot, 'slot', torch.int32), _ptr(dropped, 'dropped', torch.uint8),
                                     _ptr(counts, 'counts', torch.int32),
                                     _ptr(row_token, 'row_token', torch.int32), _ptr(xe, 'xe', dt),
                                     _stream(stream)))


def moe_dispatch_by_score(cfg, x, idx, gates, slot, dropped, counts, row_token, xe, ws, stream=None):
    """Capacity under score priority: each expert keeps its C highest-gated choices."""
    dt = torch_dtype(cfg)
    _check(_lib.moe_dispatch_by_score(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(idx, 'idx', torch.int32),
                                      _ptr(gates, 'gates', torch.float32), _ptr(slot, 'slot', torch.int32),
                                      _ptr(dropped, 'dropped', torch.uint8), _ptr(counts, 'counts', torch.int32),
                                      _ptr(row_token, 'row_token', torch.int32), _ptr(xe, 'xe', dt),
                                      _ptr(ws, 'ws'), _stream(stream)))


def moe_expert_ffn(cfg, act, groups, rows_per_group, rows, a, w_in, w_gate, b_in, w_out, b_out, F,
                   h, out, stream=None, gather=None):
    """``gather`` (optional, int32 [groups*rows_per_group]): row m of group g is
    a[gather[g*rows_per_group + m]]; ``a`` is then the whole token matrix."""
    dt = torch_dtype(cfg)
    a_rows = a.shape[0] if gather is not None else 0
    _check(_lib.moe_expert_ffn(ctypes.byref(cfg), _enum('act', act), groups, rows_per_group,
                               _ptr(rows, 'rows', torch.int32), _ptr(a, 'a', dt),
                               _ptr(gather, 'gather', torch.int32), a_rows,
                               _ptr(w_in, 'w_in', dt), _ptr(w_gate, 'w_gate', dt),
                               _ptr(b_in, 'b_in', dt), _ptr(w_out, 'w_out', dt),
                               _ptr(b_out, 'b_out', dt), F, _ptr(h, 'h', dt), _ptr(out, 'out', dt),
                               _stream(stream)))


def moe_expert_ffn_packed(cfg, act, groups, rows, total_rows, a, w_in, w_gate, b_in, w_out, b_out, F,
                          h, out, stream=None, gather=None):
    """Packed rows (dropless mode): group g's rows start at rows[0] + ... +
    rows[g-1]; ``total_rows`` bounds their sum.  ``gather`` (optional, int32):
    row m of group g is a[gather[off_g + m]]; ``a`` is then the whole token
    matrix."""
    dt = torch_dtype(cfg)
    a_rows = a.shape[0] if gather is not None else 0
    _check(_lib.moe_expert_ffn_packed(ctypes.byref(cfg), _enum('act', act), groups,
                                      _ptr(rows, 'rows', torch.int32), int(total_rows), _ptr(a, 'a', dt),
                                      _ptr(gather, 'gather', torch.int32), a_rows,
                                      _ptr(w_in, 'w_in', dt), _ptr(w_gate, 'w_gate', dt),
                                      _ptr(b_in, 'b_in', dt), _ptr(w_out, 'w_out', dt),
                                      _ptr(b_out, 'b_out', dt), F, _ptr(h, 'h', dt), _ptr(out, 'out', dt),
                                      _stream(stream)))


def moe_sequence_aux_loss(cfg, seq_len, probs, idx, loss, ws, stream=None):
    _check(_lib.moe_sequence_aux_loss(ctypes.byref(cfg), int(seq_len), _ptr(probs, 'probs', torch.float32),
                                      _ptr(idx, 'idx', torch.int32), _ptr(loss, 'loss', torch.float32),
                                      _ptr(ws, 'ws'), _stream(stream)))


def moe_update_select_bias(cfg, counts, select_bias, gamma, stream=None):
    _check(_lib.moe_update_select_bias(ctypes.byref(cfg), _ptr(counts, 'counts', torch.int32),
                                       _ptr(select_bias, 'select_bias', torch.float32), float(gamma),
                                       _stream(stream)))


def moe_combine(cfg, x, ye, shared_out, idx, gates, slot, dropped, y, stream=None):
    dt = torch_dtype(cfg)
    _check(_lib.moe_combine(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(ye, 'ye', dt),
                            _ptr(shared_out, 'shared_out', dt), _ptr(idx, 'idx', torch.int32),
                            _ptr(gates, 'gates', torch.float32), _ptr(slot, 'slot', torch.int32),
                            _ptr(dropped, 'dropped', torch.uint8), _ptr(y, 'y', dt),
                            _stream(stream)))


def moe_expert_choice(cfg, probs, row_token, sel, counts, ws, stream=None):
    """Expert-choice picks: row_token [E,C], sel [T,E] (row or -1), counts [E]."""
    _check(_lib.moe_expert_choice(ctypes.byref(cfg), _ptr(probs, 'probs', torch.float32),
                                  _ptr(row_token, 'row_token', torch.int32), _ptr(sel, 'sel', torch.int32),
                                  _ptr(counts, 'counts', torch.int32), _ptr(ws, 'ws'), _stream(stream)))


def moe_combine_expert_choice(cfg, x, ye, shared_out, probs, sel, y, stream=None):
    dt = torch_dtype(cfg)
    _check(_lib.moe_combine_expert_choice(ctypes.byref(cfg), _ptr(x, 'x', dt), _ptr(ye, 'ye', dt),
                                          _ptr(shared_out, 'shared_out', dt),
                                          _ptr(probs, 'probs', torch.float32), _ptr(sel, 'sel', torch.int32),
                                          _ptr(y, 'y', dt), _stream(stream)))


def moe_aux_losses(cfg, logits, idx, losses, ws, stream=None):
    _check(_lib.moe_aux_losses(ctypes.byref(cfg), _ptr(logits, 'logits', torch.float32),
                               _ptr(idx, 'idx', torch.int32), _ptr(losses, 'losses', torch.float32),
                               _ptr(ws, 'ws'), _stream(stream)))


_WKEYS = ('w_router', 'logit_bias', 'select_bias', 'w_in', 'w_gate', 'b_in', 'w_out', 'b_out',
          'ws_in', 'bs_in', 'ws_out', 'bs_out')
_OKEYS = ('y', 'idx', 'gates', 'slot', 'dropped', 'counts', 'losses', 'stats', 'logits', 'probs',
          'lse', 'sel')


def moe_forward(cfg, weights: dict, x, outputs: dict, ws, stream=None, events=None):
    """The whole layer.  ``weights``/``outputs``: dicts keyed like the C structs.
    ``events`` (optional): 7 hipEvent_t handles (ints) recorded at the phase
    boundaries (moe_forward_events)."""
    dt = torch_dtype(cfg)
    wd = {}
    for kk in _WKEYS:
        t = weights.get(kk)
        want = torch.float32 if kk in ('w_router', 'logit_bias', 'select_bias') else dt
        wd[kk] = _ptr(t, kk, want)
    od = {}
    want_o = dict(y=dt, idx=torch.int32, gates=torch.float32, slot=torch.int32, dropped=torch.uint8,
                  counts=torch.int32, losses=torch.float32, stats=torch.int32, logits=torch.float32,
                  probs=torch.float32, lse=torch.float32, sel=torch.int32)
    for kk in _OKEYS:
        od[kk] = _ptr(outputs.get(kk), kk, want_o[kk])
    w = moe_weights(**wd)
    o = moe_outputs(**od)
    if events is None:
        _check(_lib.moe_forward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x, 'x', dt), ctypes.byref(o),
                                _ptr(ws, 'ws'), _stream(stream)))
    else:
        ev = (ctypes.c_void_p * len(events))(*events)
        _check(_lib.moe_forward_events(ctypes.byref(cfg), ctypes.byref(w), _ptr(x, 'x', dt), ctypes.byref(o),
                                       _ptr(ws, 'ws'), _stream(stream), ev, len(events)))


def alloc_outputs(cfg, device='cuda', logits=False, probs=False, lse=False) -> dict:
    """Output tensors for moe_forward (allocation helper for callers)."""
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    o = dict(y=torch.empty(T, d, dtype=torch_dtype(cfg), device=device),
             idx=torch.empty(T, k, dtype=torch.int32, device=device),
             gates=torch.empty(T, k, dtype=torch.float32, device=device),
             slot=torch.empty(T, k, dtype=torch.int32, device=device),
             dropped=torch.empty(T, k, dtype=torch.uint8, device=device),
             counts=torch.empty(E, dtype=torch.int32, device=device),
             losses=torch.empty(2, dtype=torch.float32, device=device),
             stats=torch.empty(4, dtype=torch.int32, device=device))
    if logits:
        o['logits'] = torch.empty(T, E, dtype=torch.float32, device=device)
    if probs:
        o['probs'] = torch.empty(T, E, dtype=torch.float32, device=device)
    if lse:
        o['lse'] = torch.empty(T, dtype=torch.float32, device=device)
    if cfg.routing == MOE_EXPERT_CHOICE:
        o['sel'] = torch.empty(T, E, dtype=torch.int32, device=device)
    return o


_GKEYS = ('dx', 'dw_router', 'dlogit_bias', 'dw_in', 'dw_gate', 'db_in', 'dw_out', 'db_out', 'dws_in', 'dbs_in',
          'dws_out', 'dbs_out', 'dgates', 'dlogits')


def moe_backward_workspace_bytes(cfg: moe_config) -> int:
    return int(_lib.moe_backward_workspace_bytes(ctypes.byref(cfg)))


def backward_workspace(cfg: moe_config, device='cuda') -> torch.Tensor:
    n = moe_backward_workspace_bytes(cfg)
    if n == 0:
        raise ValueError(f'moe_backward is not built for this configuration: {cfg_summary(cfg)}')
    return torch.empty(n, dtype=torch.uint8, device=device)


def cfg_summary(cfg) -> str:
    return ', '.join(f'{n}={getattr(cfg, n)}' for n, _ in cfg._fields_)


def moe_backward(cfg, weights: dict, x, fwd_outputs: dict, fwd_ws, dy, grads: dict, bws, alpha_aux=0.0,
                 alpha_z=0.0, stream=None):
    """Backward pass of moe_forward: ``grads`` is a dict keyed like moe_grads;
    ``fwd_outputs`` and ``fwd_ws`` are the forward call's outputs and workspace."""
    dt = torch_dtype(cfg)
    wd = {kk: _ptr(weights.get(kk), kk, torch.float32 if kk in ('w_router', 'logit_bias', 'select_bias') else dt)
          for kk in _WKEYS}
    want_o = dict(y=dt, idx=torch.int32, gates=torch.float32, slot=torch.int32, dropped=torch.uint8,
                  counts=torch.int32, losses=torch.float32, stats=torch.int32, logits=torch.float32,
                  probs=torch.float32, lse=torch.float32, sel=torch.int32)
    od = {kk: _ptr(fwd_outputs.get(kk), kk, want_o[kk]) for kk in _OKEYS}
    f32 = ('dw_router', 'dlogit_bias', 'dgates', 'dlogits')
    # the per-token gradients the library writes in full: [T,k] gate
    # gradients ([T,E] under expert choice) and [T,E] logit gradients
    ng = cfg.E if cfg.routing == MOE_EXPERT_CHOICE else cfg.k
    for kk, n in (('dgates', cfg.T * ng), ('dlogits', cfg.T * cfg.E)):
        t = grads.get(kk)
        if t is not None and t.numel() != n:
            raise ValueError(f'{kk} must hold {n} float32 values for this configuration, not {t.numel()}')
    gd = {kk: _ptr(grads.get(kk), kk, torch.float32 if kk in f32 else dt) for kk in _GKEYS}
    w = moe_weights(**wd)
    o = moe_outputs(**od)
    g = moe_grads(**gd)
    _check(_lib.moe_backward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x, 'x', dt), ctypes.byref(o),
                             _ptr(fwd_ws, 'fwd_ws'), _ptr(dy, 'dy', dt), float(alpha_aux), float(alpha_z),
                             ctypes.byref(g), _ptr(bws, 'bws'), _stream(stream)))
