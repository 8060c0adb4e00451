"""Text summaries of rocprofv3 result databases (the SQLite files written by
``rocprofv3 -d DIR -o run``), for the measurement records kept with the
library.

    python -m mixture_experts_layer_20_amd.rocprof_summary trace DIR [--title T] [--command C]
    python -m mixture_experts_layer_20_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \
        --workload NAME --copy-bytes N [--command-fetch C] [--command-write C]

``trace`` prints the per-kernel table of a ``--kernel-trace --stats`` run;
with ``--skip W --take N`` it adds, for the expert GEMM launches (gate/up,
down, and the tail sums of split last rounds), the median and mean duration
over the dispatches of forward passes W .. W+N-1 in launch order (the timed
passes of ``bench.py``, after its W warm-up passes and before its phase
loop); ``--shared`` reports the shared experts' launches apart.
``counters`` takes a ``--pmc ... --kernel-trace`` run and prints, per kernel,
the mean over its dispatches of each counter and of the duration, with the
shader clock (GRBM_GUI_ACTIVE cycles per microsecond of the dispatch) and, when
collected, MFMA busy (MfmaUtil) and bf16 matrix-core work (MOPS x 512 flop).
``traffic`` takes one ``--pmc FETCH_SIZE`` run and one ``--pmc WRITE_SIZE`` run
of ``bench.py --copy-calibration`` and prints, per kernel, the average counter
value per dispatch (KiB), the calibration factor that the plain copy kernel of
known size gives (its algorithmic bytes / its counter bytes), and a JSON line
with the expert GEMM's calibrated HBM bytes per launch pair, tagged with the
SHA-256 of the GEMM code (comments and whitespace removed) it was measured on.
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, 'csrc', 'gemm.hip')
COPY_KERNEL_TAG = 'neg_kernel'      # torch's elementwise negation, used as the plain copy
GEMM_UP_ANY = r'gemm_bf16_w\d<[12]>'   # kernel-name patterns of the two expert GEMMs: gate/up
                                      # (GELU or SwiGLU) and down
GEMM_DOWN = r'gemm_bf16_w\d<0>'
XCDS = 8                            # GRBM_GUI_ACTIVE is summed over the XCDs


def gemm_code_sha256(path=GEMM_SOURCE):
    """SHA-256 of the GEMM source with comments and whitespace removed, so
    that a record stays valid across comment edits but not code edits (the
    source has no string literal holding a comment marker)."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r'/\*.*?\*/', ' ', text, flags=re.S)
    text = re.sub(r'//[^\n]*', ' ', text)
    text = ' '.join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def find_db(d):
    c = sorted(glob.glob(os.path.join(d, '**', '*results.db'), recursive=True) +
               glob.glob(os.path.join(d, '*results.db')))
    if not c:
        raise FileNotFoundError(f'no rocprofv3 results database under {d}')
    return c[0]


def kernel_table(d):
    con = sqlite3.connect(find_db(d))
    return list(con.execute('select name, total_calls, total_duration, average, percentage from top_kernels'))


def short(name, n=72):
    name = name.replace('moe::(anonymous namespace)::', '').replace('(anonymous namespace)::', '')
    return name if len(name) <= n else name[:n - 3] + '...'


def pmc_per_kernel(d, counter):
    """{kernel name: (dispatches, average value per dispatch)} for one counter."""
    con = sqlite3.connect(find_db(d))
    per = {}
    for did, kn, cn, v in con.execute(
            'select dispatch_id, kernel_name, counter_name, value from counters_collection'):
        if cn != counter:
            continue
        per.setdefault(kn, {}).setdefault(did, 0.0)
        per[kn][did] += v
    return {kn: (len(v), sum(v.values()) / len(v)) for kn, v in per.items()}


STEP_KERNELS = ((GEMM_UP_ANY, 'expert GEMM gate/up'),
                (GEMM_DOWN, 'expert GEMM down'),
                (r'tail_sum_kernel<[12]>', 'tail sum of the gate/up GEMM'),
                (r'tail_sum_kernel<0>', 'tail sum of the down GEMM'),
                (r'ksum_kernel', 'k-split sum of the down GEMM'))


def dispatch_durations(d, pattern):
    """Durations (microseconds) of the dispatches whose kernel name matches
    `pattern`, in launch order."""
    con = sqlite3.connect(find_db(d))
    rows = con.execute('select name, start, "end" from kernels order by start').fetchall()
    return [(e - b) / 1000.0 for n, b, e in rows if re.search(pattern, n)]


def _median(v):
    srt = sorted(v)
    n = len(srt)
    return srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])


def step_table(d, skip, take, shared=False):
    """{label: (dispatches, median_us, mean_us)} over the dispatches of each
    expert-GEMM kernel made by forward passes skip .. skip+take-1.  With
    shared experts a pass launches each GEMM kernel twice, the routed experts'
    launch first and the shared experts' second (no tail split there: they
    are one group of T rows), so the dispatches alternate and are reported
    apart."""
    out = {}
    for pat, label in STEP_KERNELS:
        if not shared:
            v = dispatch_durations(d, pat)[skip:skip + take]
            if v:
                out[label] = (len(v), _median(v), sum(v) / len(v))
            continue
        v = dispatch_durations(d, pat)
        if 'sum_kernel' in pat:
            # a tail or k-split sum belongs to the routed launch only
            v = v[skip:skip + take]
            parts = ((label, v),)
        else:
            v = v[2 * skip:2 * (skip + take)]
            parts = ((label + ' (routed)', v[0::2]), (label + ' (shared)', v[1::2]))
        for lab, vv in parts:
            if vv:
                out[lab] = (len(vv), _median(vv), sum(vv) / len(vv))
    return out


def cmd_trace(a):
    rows = kernel_table(a.dir)
    print(a.title)
    if a.command:
        print('command:', a.command)
    print()
    # the top_kernels view gives durations in microseconds
    print(f'{"kernel":72s} {"calls":>6s} {"total_us":>12s} {"avg_us":>10s} {"pct":>6s}')
    for name, calls, total, avg, pct in rows:
        print(f'{short(name):72s} {calls:6d} {total:12.1f} {avg:10.2f} {pct:6.2f}')
    if a.take:
        tab = step_table(a.dir, a.skip, a.take, a.shared)
        print()
        print(f'timed forward passes only: dispatches {a.skip} .. {a.skip + a.take - 1} of each kernel '
              f'(after {a.skip} warm-up passes; the phase loop excluded)')
        print(f'{"kernel":40s} {"dispatches":>10s} {"median_us":>10s} {"mean_us":>10s}')
        tot_med = tot_mean = 0.0
        for label, (n, med, mean) in tab.items():
            print(f'{label:40s} {n:10d} {med:10.2f} {mean:10.2f}')
            tot_med += med
            tot_mean += mean
        print(f'{"expert FFNs per forward pass (sum)":40s} {"":10s} {tot_med:10.2f} {tot_mean:10.2f}')
        print('json:', json.dumps({'step_kernels_us': {k: {'n': v[0], 'median': v[1], 'mean': v[2]}
                                                      for k, v in tab.items()},
                                   'expert_ffn_us_median': tot_med, 'expert_ffn_us_mean': tot_mean}))
        if a.bench_log:
            print_agreement(tab, a.bench_log)


def bench_line(path):
    """The last bench.py JSON line in a log (stdout and the profiler's lines mixed)."""
    rec = None
    for line in open(path, errors='replace'):
        if line.startswith('{"metric"'):
            rec = json.loads(line)
    if rec is None:
        raise SystemExit(f'no bench.py JSON line in {path}')
    return rec


def print_agreement(tab, log):
    """Trace sums of the timed passes against the live phase times (HIP
    events inside the same passes) that the bench line of the same run reports."""
    rec = bench_line(log)
    live = rec.get('phases_live', {})
    routed = sum(v[2] for k, v in tab.items() if '(shared)' not in k)
    shared = sum(v[2] for k, v in tab.items() if '(shared)' in k)
    print()
    print('agreement with the bench line of the same run (its JSON line in the profiled command\'s output):')
    ev = live.get('expert_ffn', {}).get('ms')
    if ev:
        print(f'  routed expert FFN: live phase (HIP events) {ev * 1000:.1f} us per pass, trace mean '
              f'{routed:.1f} us: {abs(ev * 1000 - routed) / routed * 100:.1f}% apart')
    if shared and live.get('shared_ffn', {}).get('ms'):
        sv = live['shared_ffn']['ms']
        print(f'  shared expert FFN: live phase {sv * 1000:.1f} us per pass, trace mean {shared:.1f} us: '
              f'{abs(sv * 1000 - shared) / shared * 100:.1f}% apart')
    rf = rec.get('roofline', {})
    if rf:
        print(f'  roofline.achieved {rf.get("achieved")} {rf.get("unit")} = {rf.get("frac")} of {rf.get("peak")}; '
              f'ms_per_step {rec.get("ms_per_step")}, live pass {live.get("ms_per_step")} ms')


def counters_per_kernel(d, skip_pattern=r'reduce_kernel|FillFunctor|copyBuffer|fillBuffer|elementwise'):
    """{kernel: {'n': dispatches, 'duration_us': mean, counter: mean per dispatch}}."""
    con = sqlite3.connect(find_db(d))
    try:
        dur = {did: (n, (e - b) / 1000.0) for did, n, b, e in
               con.execute('select dispatch_id, name, start, "end" from kernels')}
    except sqlite3.Error:           # counters without a kernel trace
        dur = {}
    vals = {}
    for did, kn, cn, v in con.execute('select dispatch_id, kernel_name, counter_name, value from counters_collection'):
        vals.setdefault(kn, {}).setdefault(did, {}).setdefault(cn, 0.0)
        vals[kn][did][cn] += v
    out = {}
    for kn, per in vals.items():
        if re.search(skip_pattern, kn):
            continue
        ds = [dur[did][1] for did in per if did in dur]
        row = {'n': len(per), 'duration_us': sum(ds) / len(ds) if ds else float('nan')}
        names = sorted({cn for v in per.values() for cn in v})
        for cn in names:
            xs = [v[cn] for v in per.values() if cn in v]
            row[cn] = sum(xs) / len(xs)
        out[kn] = row
    return out


def cmd_counters(a):
    tab = counters_per_kernel(a.dir)
    print(a.title)
    if a.command:
        print('command:', a.command)
    print()
    for kn, row in sorted(tab.items(), key=lambda kv: -kv[1]['duration_us'] * kv[1]['n']):
        print(f'{short(kn, 100)}')
        t = row['duration_us']
        line = [f'dispatches {row["n"]}', f'mean duration {t:.1f} us']
        if 'GRBM_GUI_ACTIVE' in row and t > 0:
            line.append(f'shader clock {row["GRBM_GUI_ACTIVE"] / XCDS / t / 1000:.3f} GHz '
                        f'(GRBM_GUI_ACTIVE over the {XCDS} XCDs / duration)')
        if 'MfmaUtil' in row:
            line.append(f'MFMA busy {row["MfmaUtil"] / 100:.3f} of SIMD cycles (MfmaUtil)')
        if 'SQ_INSTS_VALU_MFMA_MOPS_BF16' in row and t > 0:
            fl = row['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512
            line.append(f'bf16 matrix work {fl:.4g} flop = {fl / t / 1e6:.1f} TFLOP/s')
        if 'TCC_HIT_sum' in row and 'TCC_MISS_sum' in row:
            h, m = row['TCC_HIT_sum'], row['TCC_MISS_sum']
            line.append(f'L2 hit rate {h / max(1.0, h + m):.3f}')
        if 'TCP_TCC_READ_REQ_LATENCY_sum' in row and row.get('TCP_TCC_READ_REQ_sum'):
            line.append(f'L1->L2 read latency {row["TCP_TCC_READ_REQ_LATENCY_sum"] / row["TCP_TCC_READ_REQ_sum"]:.0f} '
                        f'cycles per request')
        for cn, v in row.items():
            if cn not in ('n', 'duration_us'):
                line.append(f'{cn} {v:.6g}')
        print('    ' + '; '.join(line))


def cmd_traffic(a):
    fetch = pmc_per_kernel(a.fetch_dir, 'FETCH_SIZE')
    write = pmc_per_kernel(a.write_dir, 'WRITE_SIZE')

    def pick(tab, pattern):
        hits = [(kn, v) for kn, v in tab.items() if re.search(pattern, kn)]
        if len(hits) != 1:
            raise SystemExit(f'expected one kernel matching {pattern!r}, found {[h[0] for h in hits]}')
        return hits[0][1]

    copy_f, copy_w = pick(fetch, COPY_KERNEL_TAG)[1], pick(write, COPY_KERNEL_TAG)[1]
    kib = a.copy_bytes / 1024.0
    f_fetch, f_write = kib / copy_f, kib / copy_w
    # the expert GEMM kernels: the up (or gate/up) launch, GELU or SwiGLU,
    # then down
    g2f, g2w = pick(fetch, GEMM_UP_ANY)[1], pick(write, GEMM_UP_ANY)[1]
    g0f, g0w = pick(fetch, GEMM_DOWN)[1], pick(write, GEMM_DOWN)[1]
    # the ordered sums of split last rounds and of a k-split down launch
    # belong to the launch they finish; per pair they run as often as the
    # GEMMs (dispatch-weighted mean)
    n_pair = pick(fetch, GEMM_DOWN)[0]
    sums = r'tail_sum_kernel|ksum_kernel'
    tf = sum(n * v for kn, (n, v) in fetch.items() if re.search(sums, kn)) / max(1, n_pair)
    tw = sum(n * v for kn, (n, v) in write.items() if re.search(sums, kn)) / max(1, n_pair)
    g0f, g0w = g0f + tf, g0w + tw
    print(f'HBM traffic of the expert grouped GEMM, {a.workload} workload (rocprofv3 --pmc)')
    if a.command_fetch:
        print('command (FETCH_SIZE):', a.command_fetch)
    if a.command_write:
        print('command (WRITE_SIZE):', a.command_write)
    print()
    print(f'{"kernel":60s} {"dispatches":>10s} {"FETCH_KiB":>14s} {"WRITE_KiB":>14s}')
    for kn in sorted(set(fetch) | set(write)):
        nf, vf = fetch.get(kn, (0, float('nan')))
        nw, vw = write.get(kn, (0, float('nan')))
        print(f'{short(kn, 60):60s} {max(nf, nw):10d} {vf:14.1f} {vw:14.1f}')
    print()
    print(f'calibration: the copy kernel moves {kib:.0f} KiB each way; counters read '
          f'FETCH {copy_f:.1f} KiB, WRITE {copy_w:.1f} KiB -> factors {f_fetch:.4f} (fetch), '
          f'{f_write:.4f} (write)')
    rec = {'workload': a.workload, 'gemm_code_sha256': gemm_code_sha256(),
           'fetch_bytes_per_pair': (g2f + g0f) * f_fetch * 1024, 'write_bytes_per_pair': (g2w + g0w) * f_write * 1024,
           'fetch_factor': f_fetch, 'write_factor': f_write}
    rec['traffic_bytes_per_pair'] = rec['fetch_bytes_per_pair'] + rec['write_bytes_per_pair']
    print('json:', json.dumps(rec))


def read_traffic(path, workload):
    """Calibrated bytes per launch pair from a ``traffic`` summary, or None
    when the summary is missing, for another workload, or taken on another
    version of the GEMM source."""
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith('json: '):
            rec = json.loads(line[6:])
            if rec.get('workload') == workload and rec.get('gemm_code_sha256') == gemm_code_sha256():
                return rec
    return None


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest='cmd', required=True)
    t = sub.add_parser('trace')
    t.add_argument('dir')
    t.add_argument('--title', default='rocprofv3 kernel trace')
    t.add_argument('--command', default='')
    t.add_argument('--skip', type=int, default=0, help='warm-up forward passes before the timed ones')
    t.add_argument('--take', type=int, default=0, help='timed forward passes (0: no per-step section)')
    t.add_argument('--bench-log', default='',
                   help="the profiled bench.py run's output, for the agreement of trace and live phases")
    t.add_argument('--shared', action='store_true',
                   help='the layer has shared experts (each pass launches every GEMM kernel twice)')
    cc = sub.add_parser('counters')
    cc.add_argument('dir')
    cc.add_argument('--title', default='rocprofv3 counters')
    cc.add_argument('--command', default='')
    f = sub.add_parser('traffic')
    f.add_argument('fetch_dir')
    f.add_argument('write_dir')
    f.add_argument('--workload', required=True)
    f.add_argument('--copy-bytes', type=int, required=True)
    f.add_argument('--command-fetch', default='')
    f.add_argument('--command-write', default='')
    a = p.parse_args()
    {'trace': cmd_trace, 'counters': cmd_counters, 'traffic': cmd_traffic}[a.cmd](a)


if __name__ == '__main__':
    main()
