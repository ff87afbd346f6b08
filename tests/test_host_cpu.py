"""Host-side logic on the CPU: the throughput workload's length recipe, the
FLOP model of the metric, bench.py's visible-pair count, and the rocprofv3
summary module (run on small synthetic result databases)."""
import itertools
import os
import sqlite3

import numpy as np
import pytest

import workloads
from bwd_thd_varlen_amd import rocprof_summary as rs


def test_throughput_lengths_recipe():
    """Seed 0 of the recipe (U[256, 8192] drawn until 65536 padded tokens,
    each slot padded to 64) gives these 16 sequences."""
    real, padded, _ = workloads.throughput_lengths(0)
    assert real == [7007, 5311, 4312, 2397, 2699, 581, 853, 387, 1647, 6710, 5410, 7500, 4253,
                    5070, 7960, 2880]
    assert padded == [7040, 5312, 4352, 2432, 2752, 640, 896, 448, 1664, 6720, 5440, 7552, 4288,
                      5120, 8000, 2880]
    assert sum(padded) == 65536
    assert all(p % 64 == 0 and 0 < r <= p for r, p in zip(real, padded))


def test_flop_model():
    """F_fwd = 4 d hq sum(L^2) / 2 under the causal model, F_bwd = 2.5 F_fwd:
    20.578 TFLOP per forward + backward step of the throughput workload."""
    real, _, _ = workloads.throughput_lengths(0)
    cu = np.concatenate([[0], np.cumsum(real)])
    f, b = workloads.causal_flops(cu, cu, 64, 128, True)
    assert sum(L * L for L in real) == 358846981
    assert f == 4 * 128 * 64 * 358846981 / 2
    assert f + b == 20577721278464.0
    fn, _ = workloads.causal_flops(cu, cu, 64, 128, False)
    assert fn == 2 * f


def test_visible_pairs_against_brute_force():
    import bench
    rng = np.random.default_rng(5)
    for _ in range(40):
        lq, lk = (int(x) for x in rng.integers(0, 70, size=2))
        br = sum(1 for i, j in itertools.product(range(lq), range(lk)) if j <= i + lk - lq)
        assert bench.visible_pairs(lq, lk, "bottom_right") == br
        assert bench.visible_pairs(lq, lk, False) == lq * lk
        assert bench.visible_pairs(lq, lk, True) == lq * lk / 2


def test_cpu_model_names_the_part(tmp_path):
    """A generic model name (as some virtual machines report it) still comes
    with the family / model / stepping numbers and the logical CPU count."""
    import bench
    block = ("processor\t: {i}\nvendor_id\t: AuthenticAMD\ncpu family\t: 25\nmodel\t\t: 17\n"
             "model name\t: AMD EPYC\nstepping\t: 1\nflags\t\t: fpu vme\n\n")
    path = tmp_path / "cpuinfo"
    path.write_text("".join(block.format(i=i) for i in range(3)))
    assert bench.cpu_model(str(path)) == "AMD EPYC (cpu family 25, model 17, stepping 1; 3 logical CPUs)"
    (tmp_path / "empty").write_text("")
    assert bench.cpu_model(str(tmp_path / "empty")) == "unknown"
    assert bench.cpu_model(str(tmp_path / "missing")) == "unknown"


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """The library runs on one GPU: bench.py exits with a message (status 2)
    before touching a device when asked for more."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(__file__), "..", "bench.py"),
                        *argv], capture_output=True, text=True, timeout=120,
                       env={**os.environ, **env})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _db(path, kernels=(), counters=()):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?)", kernels)
    con.execute("create view top_kernels as select name, count(*) as calls, "
                "sum(end - start) / 1000.0 as total, avg(end - start) / 1000.0 as average "
                "from kernels group by name order by total desc")
    con.execute("create table counters_collection (dispatch_id integer primary key, kernel_name text, "
                "counter_name text, value real, duration real)")
    # (kernel, counter, value) or (kernel, counter, value, dispatch duration in ns)
    con.executemany("insert into counters_collection (kernel_name, counter_name, value, duration) "
                    "values (?, ?, ?, ?)", [tuple(c) + (1000.0,) * (4 - len(c)) for c in counters])
    con.commit()
    con.close()


FWD = rs.STAGE_KERNELS["fwd"] + ", false, false>(attn::AttnParams)"
DKDV = rs.STAGE_KERNELS["dkdv"] + ", false, false, 4, 32, 0, 2, 2>(attn::AttnParams)"


def test_trace_summary(tmp_path):
    db = str(tmp_path / "t.db")
    # durations in ns: fwd 1000, 3000 (avg 2 us, median 2 us), dkdv 5000
    _db(db, kernels=[(FWD, 0, 1000), (FWD, 2000, 5000), (DKDV, 6000, 11000)])
    out = str(tmp_path / "t.md")
    rs.trace(db, out, "CMD", title="T")
    text = open(out).read()
    assert text.startswith("# Kernel trace: T")
    assert "    CMD" in text
    row = next(l for l in text.splitlines() if l.startswith("| attn::fwd_kernel"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1:6] == ["2", "2.0", "2.0", "1.0", "4.0"]   # calls, avg, median, min, total (us)
    assert cells[6] == "44.44%"


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reading half of a 1 GiB copy is scaled by 2, WRITE_SIZE by 1."""
    monkeypatch.setattr(rs, "PROFILES", str(tmp_path))
    gib_kib = (1 << 30) / 1024.0
    fetch = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2), (FWD, "FETCH_SIZE", 100.0),
             (FWD, "FETCH_SIZE", 300.0)]
    write = [("__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib), (FWD, "WRITE_SIZE", 50.0),
             (FWD, "WRITE_SIZE", 50.0)]
    _db(str(tmp_path / "f.db"), counters=fetch)
    _db(str(tmp_path / "w.db"), counters=write)
    rs.traffic(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "CF", "CW")
    text = open(tmp_path / "fwd_throughput_65k_pmc.txt").read()
    vals = dict(l.split(" = ") for l in text.splitlines() if " = " in l and not l.startswith("#"))
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert int(vals["hbm_bytes_per_launch"]) == (200 * 2 + 50) * 1024
    assert vals["kernel_source_sha256"] == rs.source_hash("fwd")
    assert not os.path.exists(tmp_path / "dq_throughput_65k_pmc.txt")   # no dq dispatches


def test_counter_summary_ratios(tmp_path):
    db = str(tmp_path / "c.db")
    _db(db, counters=[(DKDV, "SQ_WAVE_CYCLES", 1000.0), (DKDV, "SQ_WAVE_CYCLES", 3000.0),
                      (DKDV, "SQ_WAIT_INST_LDS", 200.0), (DKDV, "SQ_WAIT_INST_LDS", 200.0)])
    out = str(tmp_path / "c.txt")
    rs.counters(out, [db], ["CMD"])
    text = open(out).read()
    row = next(l for l in text.splitlines() if l.startswith("| waiting on LDS"))
    assert row.rstrip().endswith("| - | - | 10.0% |")   # 200 / 2000, dkdv only


def test_counter_summary_lds_conflicts_and_clock(tmp_path):
    """Conflict cycles per LDS instruction, and the clock from GRBM_GUI_ACTIVE
    summed over the 8 XCDs: 8 x 1.6e6 cycles in a 1 ms dispatch is 1.6 GHz."""
    db = str(tmp_path / "c.db")
    _db(db, counters=[(DKDV, "SQ_LDS_BANK_CONFLICT", 30.0, 1e6), (DKDV, "SQ_INSTS_LDS", 120.0, 1e6),
                      (DKDV, "SQ_ACTIVE_INST_LDS", 600.0, 1e6),
                      (DKDV, "GRBM_GUI_ACTIVE", 8 * 1.6e6, 1e6)])
    out = str(tmp_path / "c.txt")
    rs.counters(out, [db], ["CMD"])
    lines = open(out).read().splitlines()
    row = next(l for l in lines if l.startswith("| bank-conflict cycles per LDS instruction"))
    assert row.rstrip().endswith("| - | - | 0.25 |")
    row = next(l for l in lines if l.startswith("| shader clock"))
    assert row.rstrip().endswith("| - | - | 1.60 GHz |")


def test_counter_summary_d256_picks_the_split_kernels(tmp_path):
    """With the head-dim-256 workload the dq / dkdv columns come from the
    split kernels; d=128 kernels in the same database are not counted."""
    split_dkdv = rs.STAGE_KERNELS_D256["dkdv"] + ", false, false, false, 256>(attn::AttnParams)"
    db = str(tmp_path / "c.db")
    _db(db, counters=[(split_dkdv, "SQ_WAVE_CYCLES", 1000.0), (split_dkdv, "SQ_WAIT_INST_LDS", 250.0),
                      (DKDV, "SQ_WAVE_CYCLES", 1000.0), (DKDV, "SQ_WAIT_INST_LDS", 900.0)])
    out = str(tmp_path / "c.txt")
    rs.counters(out, [db], ["CMD"], workload="d256_65k")
    text = open(out).read()
    assert text.startswith("# Shader-sequencer counters: d256_65k workload")
    row = next(l for l in text.splitlines() if l.startswith("| waiting on LDS"))
    assert row.rstrip().endswith("| - | - | 25.0% |")


def test_source_hash_ignores_comments():
    """Comments and blank lines do not change the code hash of a stage; code does."""
    src = "int a; // one\n/* two\n three */\nint b;   \n\n"
    assert rs.code_only(src) == "int a;\nint b;"
    assert rs.code_only("int a;\nint b;") == rs.code_only(src)
    assert rs.code_only("int a;\nint c;") != rs.code_only(src)
