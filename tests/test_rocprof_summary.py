"""Host tests of the rocprofv3 summary helper: the per-kernel counter
averages, the copy-kernel calibration, and the source-hash gate that keeps
stale traffic numbers out of the bench line."""
import argparse
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
G0 = 'void moe::(anonymous namespace)::gemm_bf16_w8<0>(moe::GemmArgs)'
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


def test_traffic_of_a_gelu_layer_counts_its_k_split_sum(tmp_path):
    """A GELU layer's up launch is gemm_bf16_w8<1>; the k-split down launch's
    ordered sum (ksum_kernel) is part of the down launch's traffic."""
    g1 = 'void moe::(anonymous namespace)::gemm_bf16_w8<1>(moe::GemmArgs)'
    g0 = 'void moe::(anonymous namespace)::gemm_bf16_w8<0>(moe::GemmArgs)'
    ks = 'moe::(anonymous namespace)::ksum_kernel(moe::GemmArgs)'
    kib = (1 << 30) / 1024
    make_db(str(tmp_path / 'f'), 'FETCH_SIZE', [(1, COPY, kib), (2, g1, 700.0), (3, g0, 600.0), (4, ks, 90.0)])
    make_db(str(tmp_path / 'w'), 'WRITE_SIZE', [(1, COPY, kib), (2, g1, 30.0), (3, g0, 80.0), (4, ks, 20.0)])
    out = subprocess.run([sys.executable, '-m', 'mixture_experts_layer_20_amd.rocprof_summary', 'traffic',
                          str(tmp_path / 'f'), str(tmp_path / 'w'), '--workload', 'wl',
                          '--copy-bytes', str(1 << 30)], cwd=ROOT, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    rec = json.loads([ln for ln in out.stdout.splitlines() if ln.startswith('json: ')][0][6:])
    assert rec['fetch_bytes_per_pair'] == pytest.approx((700.0 + 600.0 + 90.0) * 1024)
    assert rec['write_bytes_per_pair'] == pytest.approx((30.0 + 80.0 + 20.0) * 1024)


def test_code_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / 'a.hip'
    a.write_text('// header\nint f(int x) {  /* note */ return x + 1; }  // tail\n')
    b = tmp_path / 'b.hip'
    b.write_text('// another header\n\nint f(int x) { return x + 1; }\n')
    c = tmp_path / 'c.hip'
    c.write_text('int f(int x) { return x + 2; }\n')
    assert R.gemm_code_sha256(str(a)) == R.gemm_code_sha256(str(b))
    assert R.gemm_code_sha256(str(a)) != R.gemm_code_sha256(str(c))


def test_timed_steps_take_the_dispatches_between_warmup_and_phase_loop(tmp_path):
    d = tmp_path / 't'
    os.makedirs(d)
    con = sqlite3.connect(os.path.join(d, 'run_results.db'))
    con.execute('create table kernels (name text, start int, "end" int)')
    con.execute('create table top_kernels (name text, total_calls int, total_duration real, average real, percentage real)')
    up = 'void moe::(anonymous namespace)::gemm_bf16_w8<2>(moe::GemmArgs)'
    down = 'void moe::(anonymous namespace)::gemm_bf16_w8<0>(moe::GemmArgs)'
    t = 0
    # 2 warm-up passes (slow), 3 timed passes, then a phase call (cold, slow)
    for dur_up, dur_dn in [(9000, 5000), (8000, 4000), (3500, 2000), (3600, 2100), (3400, 1900), (7000, 3000)]:
        con.execute('insert into kernels values (?,?,?)', (up, t, t + dur_up * 1000))
        t += dur_up * 1000 + 10
        con.execute('insert into kernels values (?,?,?)', (down, t, t + dur_dn * 1000))
        t += dur_dn * 1000 + 10
    con.commit()
    con.close()
    tab = R.step_table(str(d), 2, 3)
    assert tab['expert GEMM gate/up'] == (3, 3500.0, 3500.0)
    assert tab['expert GEMM down'] == (3, 2000.0, 2000.0)


def test_timed_steps_report_shared_expert_launches_apart(tmp_path):
    d = tmp_path / 's'
    os.makedirs(d)
    con = sqlite3.connect(os.path.join(d, 'run_results.db'))
    con.execute('create table kernels (name text, start int, "end" int)')
    con.execute('create table top_kernels (name text, total_calls int, total_duration real, average real, percentage real)')
    up = 'void moe::(anonymous namespace)::gemm_bf16_w8<1>(moe::GemmArgs)'
    down = 'void moe::(anonymous namespace)::gemm_bf16_w8<0>(moe::GemmArgs)'
    t = 0
    # per pass: routed gate/up, routed down, shared gate/up, shared down;
    # 1 warm-up pass (slow), then 2 timed passes
    for scale in (3, 1, 1):
        for name, dur in ((up, 130), (down, 110), (up, 60), (down, 55)):
            con.execute('insert into kernels values (?,?,?)', (name, t, t + scale * dur * 1000))
            t += scale * dur * 1000 + 10
    con.commit()
    con.close()
    tab = R.step_table(str(d), 1, 2, shared=True)
    assert tab['expert GEMM gate/up (routed)'] == (2, 130.0, 130.0)
    assert tab['expert GEMM gate/up (shared)'] == (2, 60.0, 60.0)
    assert tab['expert GEMM down (routed)'] == (2, 110.0, 110.0)
    assert tab['expert GEMM down (shared)'] == (2, 55.0, 55.0)


def test_agreement_reads_the_last_bench_line_of_a_mixed_log(tmp_path, capsys):
    log = tmp_path / 'run.log'
    rec = {'metric': 'm', 'ms_per_step': 0.6, 'phases_live': {'ms_per_step': 0.61, 'expert_ffn': {'ms': 0.242},
                                                             'shared_ffn': {'ms': 0.115}},
           'roofline': {'achieved': 400.0, 'unit': 'TFLOP/s', 'frac': 0.16, 'peak': 2500.0}}
    log.write_text('W profiler line\n{"metric": "old"}\n' + json.dumps(rec) + '\nW profiler end\n')
    tab = {'expert GEMM gate/up (routed)': (2, 130.0, 130.0), 'expert GEMM down (routed)': (2, 110.0, 110.0),
           'expert GEMM gate/up (shared)': (2, 60.0, 60.0), 'expert GEMM down (shared)': (2, 55.0, 55.0)}
    R.print_agreement(tab, str(log))
    out = capsys.readouterr().out
    assert 'live phase (HIP events) 242.0 us per pass, trace mean 240.0 us: 0.8% apart' in out
    assert 'shared expert FFN: live phase 115.0 us per pass, trace mean 115.0 us: 0.0% apart' in out


def test_counters_per_kernel_sum_instances_and_derive_rates(tmp_path, capsys):
    # two dispatches of one kernel, counters split over instances (summed per
    # dispatch, then averaged over dispatches), durations from the trace
    d = tmp_path / 'c'
    os.makedirs(d)
    con = sqlite3.connect(os.path.join(d, 'run_results.db'))
    con.execute('create table counters_collection (dispatch_id int, kernel_name text, counter_name text, value real)')
    con.execute('create table kernels (dispatch_id int, name text, start int, "end" int)')
    k = 'void moe::(anonymous namespace)::gemm_bf16_w8<2>(moe::GemmArgs)'
    for did, us in ((1, 1000), (2, 3000)):
        con.execute('insert into kernels values (?,?,?,?)', (did, k, 0, us * 1000))
        for _ in range(8):                             # 8 XCD instances
            con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'GRBM_GUI_ACTIVE', 200.0 * us))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'TCC_HIT_sum', 75.0))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'TCC_MISS_sum', 25.0))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'SQ_INSTS_VALU_MFMA_MOPS_BF16', 1e9))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'TCP_TCC_READ_REQ_LATENCY_sum', 3e5))
        con.execute('insert into counters_collection values (?,?,?,?)', (did, k, 'TCP_TCC_READ_REQ_sum', 1e3))
    con.commit()
    con.close()
    tab = R.counters_per_kernel(str(d))
    row = tab[k]
    assert row['n'] == 2 and row['duration_us'] == pytest.approx(2000.0)
    assert row['GRBM_GUI_ACTIVE'] == pytest.approx(8 * 200.0 * 2000)
    R.cmd_counters(argparse.Namespace(dir=str(d), title='t', command=''))
    out = capsys.readouterr().out
    assert 'shader clock 0.200 GHz' in out                     # 200 cycles per us on each XCD
    assert 'L2 hit rate 0.750' in out
    assert 'L1->L2 read latency 300 cycles per request' in out
    assert 'bf16 matrix work 5.12e+11 flop = 256.0 TFLOP/s' in out
