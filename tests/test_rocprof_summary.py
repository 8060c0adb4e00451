"""Host tests of the rocprofv3 summary helper: the per-kernel counter
averages, the copy-kernel calibration, and the source-hash gate that keeps
stale traffic numbers out of the bench line."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mixture_experts_layer_20_amd import rocprof_summary as R  # noqa: E402

G2 = 'void moe::(anonymous namespace)::gemm_bf16_w8<2>(moe::GemmArgs)'
G0 = 'void moe::(anonymous namespace)::gemm_bf16_w4<0>(moe::GemmArgs)'
COPY = 'void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>'


def make_db(d, counter, rows):
    """rows: (dispatch_id, kernel, value); each value split over two
    instances the way per-XCD counters arrive."""
    os.makedirs(d, exist_ok=True)
    con = sqlite3.connect(os.path.join(d, 'run_results.db'))
    con.execute('create table counters_collection (dispatch_id int, kernel_name text, counter_name text, value real)')
    con.execute('create table top_kernels (name text, total_calls int, total_duration real, average real, percentage real)')
    for did, kn, v in rows:
        con.execute('insert into counters_collection values (?,?,?,?)', (did, kn, counter, v / 2))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, kn, counter, v / 2))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, kn, 'OTHER', 1e9))
    con.execute('insert into top_kernels values (?,?,?,?,?)', (G2, 2, 7000.0, 3500.0, 60.0))
    con.commit()
    con.close()


def test_pmc_average_per_dispatch(tmp_path):
    make_db(str(tmp_path / 'f'), 'FETCH_SIZE', [(1, G2, 100.0), (2, G2, 300.0), (3, G0, 50.0)])
    got = R.pmc_per_kernel(str(tmp_path / 'f'), 'FETCH_SIZE')
    assert got[G2] == (2, 200.0)
    assert got[G0] == (1, 50.0)
    assert R.kernel_table(str(tmp_path / 'f'))[0][0] == G2


def test_traffic_calibration_and_hash_gate(tmp_path):
    kib = (1 << 30) / 1024
    make_db(str(tmp_path / 'f'), 'FETCH_SIZE', [(1, COPY, kib / 2), (2, G2, 1000.0), (3, G0, 500.0)])
    make_db(str(tmp_path / 'w'), 'WRITE_SIZE', [(1, COPY, kib), (2, G2, 40.0), (3, G0, 10.0)])
    out = subprocess.run([sys.executable, '-m', 'mixture_experts_layer_20_amd.rocprof_summary', 'traffic',
                          str(tmp_path / 'f'), str(tmp_path / 'w'), '--workload', 'wl',
                          '--copy-bytes', str(1 << 30)], cwd=ROOT, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    rec = json.loads([ln for ln in out.stdout.splitlines() if ln.startswith('json: ')][0][6:])
    assert rec['fetch_factor'] == pytest.approx(2.0) and rec['write_factor'] == pytest.approx(1.0)
    assert rec['fetch_bytes_per_pair'] == pytest.approx(1500.0 * 2.0 * 1024)
    assert rec['write_bytes_per_pair'] == pytest.approx(50.0 * 1024)
    assert rec['gemm_code_sha256'] == R.gemm_code_sha256()
    path = tmp_path / 'summary.txt'
    path.write_text(out.stdout)
    assert R.read_traffic(str(path), 'wl')['traffic_bytes_per_pair'] == pytest.approx((3000.0 + 50.0) * 1024)
    assert R.read_traffic(str(path), 'other') is None
    # a summary taken on another version of the GEMM source is not used
    stale = dict(rec, gemm_code_sha256='0' * 64)
    path.write_text('json: ' + json.dumps(stale) + '\n')
    assert R.read_traffic(str(path), 'wl') is None
    assert R.read_traffic(str(tmp_path / 'missing.txt'), 'wl') is None


def test_code_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / 'a.hip'
    a.write_text('// header\nint f(int x) {  /* note */ return x + 1; }  // tail\n')
    b = tmp_path / 'b.hip'
    b.write_text('// another header\n\nint f(int x) { return x + 1; }\n')
    c = tmp_path / 'c.hip'
    c.write_text('int f(int x) { return x + 2; }\n')
    assert R.gemm_code_sha256(str(a)) == R.gemm_code_sha256(str(b))
    assert R.gemm_code_sha256(str(a)) != R.gemm_code_sha256(str(c))
