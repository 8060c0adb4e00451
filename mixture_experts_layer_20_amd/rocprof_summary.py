"""Text summaries of rocprofv3 result databases (the SQLite files written by
``rocprofv3 -d DIR -o run``), for the measurement records kept with the
library.

    python -m mixture_experts_layer_20_amd.rocprof_summary trace DIR [--title T] [--command C]
    python -m mixture_experts_layer_20_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \
        --workload NAME --copy-bytes N [--command-fetch C] [--command-write C]

``trace`` prints the per-kernel table of a ``--kernel-trace --stats`` run.
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
GEMM_UP = r'gemm_bf16_w\d<2>'       # kernel-name patterns of the two expert GEMMs
GEMM_DOWN = r'gemm_bf16_w\d<0>'


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


def cmd_traffic(a):
    fetch = pmc_per_kernel(a.fetch_dir, 'FETCH_SIZE')
    write = pmc_per_kernel(a.write_dir, 'WRITE_SIZE')

    def pick(tab, pattern):
        hits = [(kn, v) for kn, v in tab.items() if re.search(pattern, kn)]
        if len(hits) != 1:
            raise SystemExit(f'expected one kernel matching {tag!r}, found {[h[0] for h in hits]}')
        return hits[0][1]

    copy_f, copy_w = pick(fetch, COPY_KERNEL_TAG)[1], pick(write, COPY_KERNEL_TAG)[1]
    kib = a.copy_bytes / 1024.0
    f_fetch, f_write = kib / copy_f, kib / copy_w
    # the expert GEMM kernels (either workgroup size): SwiGLU up/gate, then down
    g2f, g2w = pick(fetch, GEMM_UP)[1], pick(write, GEMM_UP)[1]
    g0f, g0w = pick(fetch, GEMM_DOWN)[1], pick(write, GEMM_DOWN)[1]
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
    f = sub.add_parser('traffic')
    f.add_argument('fetch_dir')
    f.add_argument('write_dir')
    f.add_argument('--workload', required=True)
    f.add_argument('--copy-bytes', type=int, required=True)
    f.add_argument('--command-fetch', default='')
    f.add_argument('--command-write', default='')
    a = p.parse_args()
    cmd_trace(a) if a.cmd == 'trace' else cmd_traffic(a)


if __name__ == '__main__':
    main()
