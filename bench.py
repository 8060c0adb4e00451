"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--phase-reps R] [--dropless]
                    [--routing token|expert] [--priority rank|token|score] [--backward]
                    [--save-preact | --no-save-preact] [--graph]

A step is one whole forward pass of the layer (router, capacity, dispatch,
routed and shared expert FFNs, combine, losses) over one batch of T synthetic
tokens that are already resident in HBM, through moe_forward on torch's
current stream.  `value` is tokens per second over the K timed steps.

After the headline loop, K more steps run through moe_forward_events, which
records HIP events on the library's stream at the boundaries of each phase of
the same forward pass; their per-step durations (`phases_live`, caches warm
as in the layer) give
  * roofline: the expert grouped GEMM (the dominant kernel: its gate/up and
    down launches) against the bf16 MFMA peak, from algorithmic FLOPs
    2 * kept_assignments * (3 or 2) * d * d_ff, averaged over the K steps.
The run also times each phase through the public entry points (moe_route,
moe_dispatch, moe_expert_ffn, moe_combine) after flushing L2 and the MALL
(`phases`, cold caches), giving router, dispatch and combine against the HBM
peak from their algorithmic bytes, and
  * cpu_baseline: the CPU oracle (tests' reference implementation) timed on a
    bounded sample of the same workload, with the host's core count and model.
Prints ONE JSON line.  `--cpu-baseline-all` instead times the oracle on every
workload (bounded samples) and the pure-Python brute force on the tiny one,
and prints a table.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (vector / matrix)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = 'MoE layer tokens/sec at 1 GPU; expert-GEMM % MFMA peak; route/combine % HBM'


def parse():
    p = argparse.ArgumentParser()
    p.add_argument('--gpus', type=int, default=1)
    p.add_argument('--steps', type=int, default=20)
    p.add_argument('--warmup', type=int, default=5)
    p.add_argument('--workload', default='mixtral_8x_top2')
    p.add_argument('--no-cpu-baseline', action='store_true')
    p.add_argument('--cpu-sample-tokens', type=int, default=0)
    p.add_argument('--phase-reps', type=int, default=10)
    p.add_argument('--dropless', action='store_true',
                   help='dropless mode: no capacity limit, expert rows packed without padding')
    p.add_argument('--routing', choices=('token', 'expert'), default='token',
                   help='token choice (each token its top-k experts) or expert choice (each expert its '
                        'top-C tokens)')
    p.add_argument('--priority', choices=('rank', 'token', 'score'), default='rank',
                   help='capacity queue order: rank-major (GShard), token-major, or by router score '
                        '(batch-prioritised)')
    p.add_argument('--backward', action='store_true',
                   help='also time moe_backward (the gradients of the same layer) as a phase')
    p.add_argument('--save-preact', action='store_true',
                   help='the forward pass keeps the expert pre-activations for the backward pass '
                        '(the default with --backward)')
    p.add_argument('--no-save-preact', action='store_true',
                   help='with --backward: recompute the pre-activations in the backward pass instead')
    p.add_argument('--graph', action='store_true',
                   help='capture one moe_forward into a HIP graph and time its replays')
    p.add_argument('--copy-calibration', action='store_true',
                   help='finish with a plain copy kernel of known size (for calibrating HBM byte counters)')
    p.add_argument('--cpu-baseline-all', action='store_true',
                   help='time the CPU oracle on every workload (bounded samples) and the brute force on the '
                        'tiny one; no GPU work')
    p.add_argument('--yardstick-shapes', default=None,
                   help='with --vendor-yardstick: comma-separated MxNxK shapes')
    p.add_argument('--vendor-yardstick', action='store_true',
                   help='time the vendor dense GEMM (through torch) on the Mixtral-shaped expert GEMMs, for '
                        'comparison only; no MoE layer')
    args = p.parse_args()
    if args.save_preact and args.no_save_preact:
        p.error('--save-preact and --no-save-preact exclude each other')
    # a training step keeps the pre-activations unless asked not to
    args.save_preact = args.save_preact or (args.backward and not args.no_save_preact)
    return args


YARDSTICK_SHAPES = '16384x28672x4096,16384x4096x14336,2048x28672x4096,2048x4096x14336'


def vendor_yardstick(steps, shapes=YARDSTICK_SHAPES):
    """torch's dense bf16 GEMM (the vendor library) on the shapes of the
    Mixtral-shaped layer's expert GEMMs (M x N x K): all 16,384 kept rows at
    once, and one expert's 2,048 rows; random normal operands, steady state."""
    import torch
    for M, N, K in (tuple(int(v) for v in sh.split('x')) for sh in shapes.split(',')):
        g = torch.Generator('cuda').manual_seed(7)
        a = torch.randn(M, K, device='cuda', dtype=torch.bfloat16, generator=g)
        b = (torch.randn(N, K, device='cuda', dtype=torch.bfloat16, generator=g) / 64).contiguous()
        for _ in range(5):
            c = a @ b.t()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            c = a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        print(f'vendor GEMM {M}x{N}x{K}: {ms:.3f} ms, {2 * M * N * K / ms / 1e9:.1f} TFLOP/s '
              f'({2 * M * N * K / ms / 1e9 / PEAK_BF16_TFLOPS:.3f} of peak)', flush=True)
        del a, b, c


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded (the library
    records them on its stream)."""

    def __init__(self):
        import ctypes
        path = None
        with open('/proc/self/maps') as f:
            for line in f:
                if 'libamdhip64' in line:
                    path = line.split()[-1]
                    break
        self.ct = ctypes
        self.lib = ctypes.CDLL(path or 'libamdhip64.so')
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        h = self.ct.c_void_p()
        if self.lib.hipEventCreate(self.ct.byref(h)) != 0:
            raise RuntimeError('hipEventCreate failed')
        self.made.append(h.value)
        return h.value

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(out), a, b) != 0:
            raise RuntimeError('hipEventElapsedTime failed')
        return float(out.value)

    def close(self):
        for h in self.made:
            self.lib.hipEventDestroy(h)
        self.made = []


COPY_BYTES = 1 << 30           # bytes read and bytes written by the calibration copy


def main():
    args = parse()
    if args.cpu_baseline_all:
        cpu_baseline_all()
        return
    if args.vendor_yardstick:
        vendor_yardstick(max(1, args.steps), args.yardstick_shapes or YARDSTICK_SHAPES)
        return
    if args.gpus != 1:
        print(json.dumps({'error': 'one GPU only: the MoE layer is measured on a single MI355X (the '
                                   'multi-GPU sharding is designed, not built); --gpus must be 1'}), flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_20_amd as moe
    import synth

    def log(*a):
        print('[bench]', *a, file=sys.stderr, flush=True)

    w = synth.WORKLOADS[args.workload]
    ec = args.routing == 'expert'
    if ec and args.dropless:
        print(json.dumps({'error': 'expert-choice routing has no dropless mode'}), flush=True)
        sys.exit(2)
    dev = 'cuda'
    t0 = time.time()
    inp = synth.router_inputs(w)
    cfg = moe.config_from_workload(w, dropless=args.dropless, routing=args.routing, priority=args.priority,
                                   save_preact=args.save_preact)
    C = moe.moe_validate(cfg)
    x = synth.to_torch(inp['x'], dev)
    weights = dict(w_router=synth.to_torch(inp['w_router'], dev),
                   logit_bias=synth.to_torch(inp['logit_bias'], dev),
                   select_bias=synth.to_torch(inp['select_bias'], dev))
    dt = moe.torch_dtype(cfg)
    # expert weights generated one expert at a time straight into device tensors
    F, d, E = w.d_ff, w.d, w.E
    names = ('w_gate', 'w_up', 'w_out') if w.act == 'swiglu' else ('w_in', 'b_in', 'w_out', 'b_out')
    host_ex = {}
    for e in range(E):
        ew = synth.expert_weights(w, e)
        for kk in names:
            v = ew[kk]
            if kk in ('b_in', 'b_out') and w.dtype == 'bf16':
                v = synth.bf16_bits(v)
            if kk not in host_ex:
                host_ex[kk] = torch.empty((E,) + v.shape, dtype=dt, device=dev)
            host_ex[kk][e].copy_(synth.to_torch(v, dev))
    if w.act == 'swiglu':
        weights.update(w_gate=host_ex['w_gate'], w_in=host_ex['w_up'], w_out=host_ex['w_out'])
    else:
        weights.update(host_ex)
    if w.n_shared:
        sh = synth.all_expert_weights(w, shared=True)
        bs_in = np.concatenate(list(sh['b_in']))
        bs_out = sh['b_out'].sum(0).astype(np.float32)
        if w.dtype == 'bf16':
            bs_in, bs_out = synth.bf16_bits(bs_in), synth.bf16_bits(bs_out)
        weights.update(ws_in=synth.to_torch(np.concatenate(list(sh['w_in']), 0), dev),
                       ws_out=synth.to_torch(np.concatenate(list(sh['w_out']), 1), dev),
                       bs_in=synth.to_torch(bs_in, dev), bs_out=synth.to_torch(bs_out, dev))
    out = moe.alloc_outputs(cfg, dev)
    ws = moe.workspace(cfg, dev)
    torch.cuda.synchronize()
    log(f'inputs ready in {time.time() - t0:.1f}s: {w.name} T={w.T} d={d} E={E} k={w.k} F={F} C={C}')

    # ---------------------------------------------------------------- headline
    step = lambda: moe.moe_forward(cfg, weights, x, out, ws)
    if args.graph:
        # the library enqueues kernels only, so one call captures whole
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            moe.moe_forward(cfg, weights, x, out, ws, stream=gs)
        torch.cuda.current_stream().wait_stream(gs)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            moe.moe_forward(cfg, weights, x, out, ws, stream=gs)
        step = graph.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = 1e3 * elapsed / max(1, args.steps)
    tokens_per_s = w.T * args.steps / elapsed
    stats = out['stats'].cpu().tolist()
    kept, n_dropped, fallback, pad = stats
    log(f'forward: {ms:.3f} ms/step, {tokens_per_s:,.0f} tokens/s, kept {kept}, dropped {n_dropped}, '
        f'fallback {fallback}')

    # ---------------------------------------------------------------- live phases
    # K more forward passes, each recording events at its phase boundaries
    live_names = ('route', 'dispatch', 'expert_ffn', 'shared_ffn', 'combine', 'losses')
    hev = HipEvents()
    evs = [[hev.create() for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_live = time.perf_counter()
    for sev in evs:
        moe.moe_forward(cfg, weights, x, out, ws, events=sev)
    torch.cuda.synchronize()
    live_ms_step = 1e3 * (time.perf_counter() - t_live) / max(1, args.steps)
    live = {nm: [hev.ms(sev[i], sev[i + 1]) for sev in evs] for i, nm in enumerate(live_names)}
    live['kernels'] = [hev.ms(sev[0], sev[6]) for sev in evs]
    hev.close()
    log(f'live: {live_ms_step:.3f} ms/step; ' + ', '.join(
        f'{nm} {np.mean(v):.4g} ms' for nm, v in live.items()))

    # ---------------------------------------------------------------- phases
    T, k = w.T, w.k
    b = 2 if w.dtype == 'bf16' else 4
    idx, gates = out['idx'], out['gates']
    slot = torch.empty_like(out['slot'])
    dropped = torch.empty_like(out['dropped'])
    counts = torch.empty_like(out['counts'])
    # expert rows: E x C (capacity), or T*k packed back to back (dropless)
    xrows = T * k if args.dropless else E * C
    row_token = torch.empty(xrows, dtype=torch.int32, device=dev)
    h = torch.empty(xrows, F, dtype=dt, device=dev)
    ye = torch.empty(xrows, d, dtype=dt, device=dev)
    y = torch.empty_like(out['y'])
    fs = w.n_shared * w.d_ff_shared
    hs = torch.empty(T, fs, dtype=dt, device=dev) if fs else None
    s_out = torch.empty(T, d, dtype=dt, device=dev) if fs else None
    # cache flush between phase repetitions: a read of 512 MiB (twice the
    # MALL).  Reading rather than writing leaves no dirty lines whose
    # write-back would land inside the measured kernel.
    flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    ph = {'route': [], 'dispatch': [], 'expert_ffn': [], 'shared_ffn': [], 'combine': []}
    probs = torch.empty(T, E, dtype=torch.float32, device=dev) if ec else None
    sel = torch.empty(T, E, dtype=torch.int32, device=dev) if ec else None

    def timed(name, fn):
        torch.sum(flush, dim=0, out=flush_sink)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        z.record()
        z.synchronize()
        ph[name].append(a.elapsed_time(z))

    kept_rows = torch.empty(E, dtype=torch.int32, device=dev)
    for rep in range(args.phase_reps + 1):
        timed('route', lambda: moe.moe_route(cfg, x, weights['w_router'], weights['logit_bias'],
                                             weights['select_bias'], None, probs, idx, gates, None, ws))
        if ec:
            # every expert's top-C tokens (the 'dispatch' phase of expert choice)
            timed('dispatch', lambda: moe.moe_expert_choice(cfg, probs, row_token, sel, counts, ws))
        else:
            # capacity slots and the token list of every expert (the layer gathers
            # token rows inside the expert GEMM, so nothing is copied here)
            if args.priority == 'score' and not args.dropless:
                timed('dispatch', lambda: moe.moe_dispatch_by_score(cfg, None, idx, gates, slot, dropped, counts,
                                                                    row_token, None, ws))
            else:
                timed('dispatch', lambda: moe.moe_dispatch(cfg, None, idx, slot, dropped, counts, row_token,
                                                           None, ws))
        torch.clamp(counts, max=C, out=kept_rows)
        if args.dropless:
            timed('expert_ffn', lambda: moe.moe_expert_ffn_packed(
                cfg, w.act, E, counts, T * k, x, weights['w_in'], weights.get('w_gate'), weights.get('b_in'),
                weights['w_out'], weights.get('b_out'), F, h, ye, gather=row_token))
        elif w.act == 'swiglu':
            timed('expert_ffn', lambda: moe.moe_expert_ffn(cfg, 'swiglu', E, C, kept_rows, x, weights['w_in'],
                                                           weights['w_gate'], None, weights['w_out'], None,
                                                           F, h, ye, gather=row_token))
        else:
            timed('expert_ffn', lambda: moe.moe_expert_ffn(cfg, 'gelu', E, C, kept_rows, x, weights['w_in'],
                                                           None, weights.get('b_in'), weights['w_out'],
                                                           weights.get('b_out'), F, h, ye, gather=row_token))
        if fs:
            timed('shared_ffn', lambda: moe.moe_expert_ffn(cfg, 'gelu', 1, T, None, x, weights['ws_in'], None,
                                                           weights['bs_in'], weights['ws_out'], weights['bs_out'],
                                                           fs, hs, s_out))
        if ec:
            timed('combine', lambda: moe.moe_combine_expert_choice(cfg, x, ye, s_out, probs, sel, y))
        else:
            timed('combine', lambda: moe.moe_combine(cfg, x, ye, s_out, idx, gates, slot, dropped, y))
    med = {kk: float(np.median(v[1:])) for kk, v in ph.items() if v}
    n_kept = int(torch.clamp(counts, max=C).sum().item())
    any_kept = (sel >= 0).any(dim=1) if ec else (dropped == 0).any(dim=1)
    n_tok_kept = int(any_kept.sum().item())
    n_fb = T - n_tok_kept
    mult = 3 if w.act == 'swiglu' else 2
    ffn_flops = 2.0 * n_kept * mult * d * F
    sh_flops = 2.0 * T * 2 * d * fs
    bytes_route = T * d * b + d * E * 4 + T * k * 8 + ((T + 31) // 32) * (E + 1) * 8 + (T * E * 4 if ec else 0)
    if ec:
        # probabilities in; sel and the picked tokens out
        bytes_dispatch = T * E * 4 + T * E * 4 + n_kept * 4
        bytes_combine = (n_kept * d * b + (0 if fs else n_fb * d * b) + (T * d * b if fs else 0) + T * d * b
                         + T * E * 8)
    else:
        # slots only: idx in; slot, dropped, row_token out (+ the tile histograms)
        bytes_dispatch = T * k * 4 + T * k * 5 + n_kept * 4
        bytes_combine = (n_kept * d * b + (0 if fs else n_fb * d * b) + (T * d * b if fs else 0) + T * d * b
                         + T * k * 13)
    peak = PEAK_BF16_TFLOPS if w.dtype == 'bf16' else PEAK_F32_TFLOPS

    def gbs(nbytes, ms_):
        return nbytes / (ms_ * 1e-3) / 1e9

    phases = {
        'route': {'ms': med['route'], 'GB/s': gbs(bytes_route, med['route']),
                  'hbm_frac': gbs(bytes_route, med['route']) / PEAK_HBM_GBS, 'bytes': bytes_route},
        'dispatch': {'ms': med['dispatch'], 'GB/s': gbs(bytes_dispatch, med['dispatch']),
                     'hbm_frac': gbs(bytes_dispatch, med['dispatch']) / PEAK_HBM_GBS, 'bytes': bytes_dispatch},
        'expert_ffn': {'ms': med['expert_ffn'], 'TFLOP/s': ffn_flops / (med['expert_ffn'] * 1e-3) / 1e12,
                       'mfma_frac': ffn_flops / (med['expert_ffn'] * 1e-3) / 1e12 / peak, 'flops': ffn_flops},
        'combine': {'ms': med['combine'], 'GB/s': gbs(bytes_combine, med['combine']),
                    'hbm_frac': gbs(bytes_combine, med['combine']) / PEAK_HBM_GBS, 'bytes': bytes_combine},
    }
    if fs:
        phases['shared_ffn'] = {'ms': med['shared_ffn'], 'TFLOP/s': sh_flops / (med['shared_ffn'] * 1e-3) / 1e12,
                                'mfma_frac': sh_flops / (med['shared_ffn'] * 1e-3) / 1e12 / peak,
                                'flops': sh_flops}
    for kk, v in phases.items():
        log(f'phase {kk}: ' + ', '.join(f'{a}={bb:.4g}' if isinstance(bb, float) else f'{a}={bb}'
                                      for a, bb in v.items()))
    # the dominant kernel's time: the live expert-FFN phase of the timed
    # forward passes (both grouped GEMM launches), averaged over the K steps
    ffn_live_ms = float(np.mean(live['expert_ffn']))
    ach = ffn_flops / (ffn_live_ms * 1e-3) / 1e12
    # HBM bytes per launch pair from the committed FETCH_SIZE / WRITE_SIZE
    # counter runs, if they were taken on this version of the GEMM source
    from mixture_experts_layer_20_amd import rocprof_summary
    wl_key = (w.name + ('_dropless' if args.dropless else '') + ('_expert_choice' if ec else '')
              + ('' if args.priority == 'rank' else '_' + args.priority + '_priority'))
    rec = rocprof_summary.read_traffic(os.path.join(ROOT, 'profiles', f'gemm_traffic_{wl_key}.txt'), wl_key)
    roofline = {'kernel': 'expert grouped GEMM (gate/up launch + down launch)',
                'bound': 'mfma', 'achieved': round(ach, 2), 'peak': peak, 'unit': 'TFLOP/s',
                'frac': round(ach / peak, 4),
                'ms_per_launch_pair': round(ffn_live_ms, 5),
                'timing': f'HIP events around the expert FFN inside each of the {args.steps} timed forward '
                          f'passes (moe_forward_events), mean',
                'traffic': round(rec['traffic_bytes_per_pair']) if rec else None,
                'algorithmic': f'2*kept*{mult}*d*d_ff = {ffn_flops:.4e} flop per launch pair, '
                               f'kept={n_kept}'}
    if rec:
        roofline['traffic_note'] = (f'HBM bytes per launch pair: fetch {rec["fetch_bytes_per_pair"]:.4g} + write '
                                    f'{rec["write_bytes_per_pair"]:.4g}, counters scaled by a plain copy kernel '
                                    f'(factors {rec["fetch_factor"]:.3f} / {rec["write_factor"]:.3f})')

    live_bytes = {'route': bytes_route, 'dispatch': bytes_dispatch, 'combine': bytes_combine}
    live_phases = {'ms_per_step': round(live_ms_step, 4),
                   'kernels_ms_per_step': round(float(np.mean(live['kernels'])), 5)}
    for nm in live_names:
        ms_ = float(np.mean(live[nm]))
        ent = {'ms': round(ms_, 5)}
        if nm in live_bytes and ms_ > 0:
            ent['GB/s'] = round(gbs(live_bytes[nm], ms_), 2)
            ent['hbm_frac'] = round(gbs(live_bytes[nm], ms_) / PEAK_HBM_GBS, 5)
        if nm == 'expert_ffn':
            ent['TFLOP/s'] = round(ach, 2)
            ent['mfma_frac'] = round(ach / peak, 5)
        live_phases[nm] = ent

    if args.backward:
        phases['backward'] = time_backward(moe, cfg, w, weights, x, args, ffn_flops, peak, log)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample_tokens, log, dropless=args.dropless, routing=args.routing,
                           priority=args.priority)

    line = {'metric': METRIC, 'value': round(tokens_per_s, 1), 'unit': 'tokens/s', 'n_gpus': 1,
            'steps': args.steps, 'warmup': args.warmup, 'ms_per_step': round(ms, 4),
            'higher_is_better': True, 'scaling': 'weak', 'vs_baseline': None, 'dtype': w.dtype,
            'data': 'synthetic (seeded; random-init weights of the named shape)',
            'config': {'workload': w.name, 'T': w.T, 'd': d, 'E': E, 'k': k, 'd_ff': F, 'act': w.act,
                       'score': w.score, 'capacity_factor': w.cf, 'capacity': C,
                       'n_shared': w.n_shared, 'kept_assignments': kept, 'dropped_assignments': n_dropped,
                       'dropless': bool(args.dropless), 'routing': args.routing, 'priority': args.priority,
                       'save_preact': bool(args.save_preact), 'graph': bool(args.graph)},
            'roofline': roofline,
            'phases': {kk: {a: (round(bb, 5) if isinstance(bb, float) else bb) for a, bb in v.items()}
                       for kk, v in phases.items()},
            'phases_live': live_phases,
            'cpu_baseline': cpu}
    print(json.dumps(line), flush=True)


def time_backward(moe, cfg, w, weights, x, args, ffn_flops, peak, log):
    """moe_backward of the layer after one moe_forward, timed over --steps
    calls with HIP events on the library's stream.  Algorithmic work: twice
    the forward's expert matmul flops (input and weight gradients; the
    backward pass also recomputes the expert pre-activations, which is not
    counted)."""
    import torch
    T, d, E, F, k = w.T, w.d, w.E, w.d_ff, w.k
    out = moe.alloc_outputs(cfg, 'cuda', logits=True)
    ws = moe.workspace(cfg, 'cuda')
    moe.moe_forward(cfg, weights, x, out, ws)
    bf = moe.torch_dtype(cfg)
    grads = dict(dx=torch.empty(T, d, dtype=bf, device='cuda'), dw_router=torch.empty(d, E, device='cuda'),
                 dw_in=torch.empty(E, F, d, dtype=bf, device='cuda'), dw_out=torch.empty(E, d, F, dtype=bf, device='cuda'))
    if w.act == 'swiglu':
        grads['dw_gate'] = torch.empty(E, F, d, dtype=bf, device='cuda')
    fs = w.n_shared * w.d_ff_shared
    if fs:
        grads.update(dws_in=torch.empty(fs, d, dtype=bf, device='cuda'),
                     dws_out=torch.empty(d, fs, dtype=bf, device='cuda'))
    bws = moe.backward_workspace(cfg, 'cuda')
    dy = torch.randn(T, d, device='cuda', generator=torch.Generator('cuda').manual_seed(5)).to(bf)
    for _ in range(max(1, args.warmup)):
        moe.moe_backward(cfg, weights, x, out, ws, dy, grads, bws, 0.01, 0.001)
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        moe.moe_backward(cfg, weights, x, out, ws, dy, grads, bws, 0.01, 0.001)
    z.record()
    z.synchronize()
    ms = a.elapsed_time(z) / max(1, args.steps)
    flops = 2.0 * ffn_flops
    tf = flops / (ms * 1e-3) / 1e12
    log(f'phase backward: ms={ms:.4g}, TFLOP/s={tf:.4g} (algorithmic 2x forward expert flops), '
        f'workspace {bws.numel() / 2**30:.2f} GiB')
    return {'ms': ms, 'TFLOP/s': tf, 'mfma_frac': tf / peak, 'flops': flops,
            'workspace_bytes': int(bws.numel())}


def cpu_baseline(w, sample_tokens, log, dropless=False, routing='token', priority='rank'):
    """The oracle as it stands, on the first `sample_tokens` tokens of the same
    workload taken as a batch of their own (routing, capacity, every expert
    FFN and the combine, in float64 on the host cores)."""
    import numpy as np
    import synth
    from oracle import moe as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get('num_threads', 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    n = sample_tokens or {'mixtral_8x_top2': 8192, 'sigmoid_stress': 1024}.get(w.name, min(w.T, 4096))
    ws_ = w.with_(T=n)
    inp = synth.router_inputs(w)
    inp = dict(inp, x=inp['x'][:n])
    experts = [synth.expert_weights(w, e) for e in range(w.E)]
    shared = [synth.expert_weights(w, s, shared=True) for s in range(w.n_shared)] or None
    t = time.perf_counter()
    O.moe_forward(ws_, inp, lambda e: experts[e], (lambda s: shared[s]) if shared else None,
                  dropless=dropless, routing=routing, priority=priority)
    el = time.perf_counter() - t
    host = host_info()
    log(f'cpu oracle: {n} tokens in {el:.1f}s on {threads} threads ({host["nproc"]} logical CPUs, '
        f'{host["cpu_model"]})')
    return {'value': round(n / el, 2), 'unit': 'tokens/s', 'cores': threads, 'kind': 'oracle',
            'nproc': host['nproc'], 'cpu_model': host['cpu_model'],
            'sample': f'the first {n} tokens of the {w.name} workload as one batch (T={n}, same d, E, k, '
                      f'd_ff and capacity factor; {routing} choice{", dropless" if dropless else ""}); '
                      f'routing, capacity, all expert FFNs and the combine in float64 numpy on {threads} '
                      f'BLAS threads; wall {el:.1f}s'}


def host_info():
    """Logical CPUs this process may use and the CPU model name."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except Exception:
        nproc = os.cpu_count() or 1
    model = 'unknown'
    try:
        with open('/proc/cpuinfo') as f:
            for line in f:
                if line.startswith('model name'):
                    model = line.split(':', 1)[1].strip()
                    break
    except OSError:
        pass
    return {'nproc': nproc, 'cpu_model': model}


# bounded samples for the all-workload oracle table: the first n tokens of each
# workload as a batch of its own (the 128-expert stress layer on 1,024 tokens)
CPU_SAMPLES = {'tiny_f32': 64, 'switch_top1_skewed': 4096, 'mixtral_8x_top2': 8192,
               'deepseekmoe_fine': 16384, 'sigmoid_stress': 1024}


def cpu_baseline_all():
    """The oracle (float64 numpy) on every workload, median of 3 where a run
    takes under 20 s, and the pure-Python brute force on the tiny layer; one
    line per workload, then a JSON summary."""
    import numpy as np
    import synth
    from oracle import brute as B
    host = host_info()
    print(f'host: {host["nproc"]} logical CPUs, {host["cpu_model"]}', flush=True)
    rows = {}
    for name, n in CPU_SAMPLES.items():
        w = synth.WORKLOADS[name]
        reps = []
        for _ in range(3):
            r = cpu_baseline(w, n, lambda *a: None)
            reps.append(r)
            if float(r['sample'].rsplit('wall ', 1)[1].rstrip('s')) > 20:
                break
        vals = sorted(r['value'] for r in reps)
        rows[name] = {'tokens_per_s': vals[len(vals) // 2], 'runs': len(reps), 'sample_tokens': n,
                      'of_T': w.T, 'threads': reps[0]['cores']}
        print(f'{name:22s} oracle {vals[len(vals) // 2]:>12,.1f} tokens/s  (first {n} of {w.T} tokens, '
              f'median of {len(reps)}, {reps[0]["cores"]} BLAS threads)', flush=True)
    from oracle import moe as O
    w = synth.WORKLOADS['tiny_f32']
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    tol = (lambda v: synth.as_f32(v).astype(np.float64).tolist())
    x = tol(inp['x'])
    wr = inp['w_router'].astype(np.float64).tolist()
    experts = [{kk: tol(v[e]) for kk, v in ex.items()} for e in range(w.E)]
    C = O.capacity(w.T, w.k, w.E, w.cf)
    t = time.perf_counter()
    B.forward(x, wr, None, None, experts, [], k=w.k, act=w.act, score=w.score, renormalize=w.renormalize,
              C=C, dtype=w.dtype)
    el = time.perf_counter() - t
    rows['tiny_f32_brute_force'] = {'seconds': round(el, 3), 'tokens_per_s': round(w.T / el, 1)}
    print(f'{"tiny_f32":22s} brute force (pure Python, one thread): {el:.3f} s = {w.T / el:,.1f} tokens/s',
          flush=True)
    print(json.dumps({'host': host, 'oracle': rows}), flush=True)


if __name__ == '__main__':
    main()
