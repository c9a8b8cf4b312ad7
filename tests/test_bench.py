"""bench.py keeps its contract: one GPU only, one JSON line with the metric, the
roofline and the CPU-oracle baseline; algorithmic byte counts per workload.
The GPU tests run short benches in this process (bench.main with an argument
list) and check the line."""
import json

import pytest

import bench
import synth


def run_bench(capsys, *args):
    """bench.main(args) in this process; returns its JSON lines."""
    capsys.readouterr()
    bench.main(list(args))
    out = capsys.readouterr().out
    return [x for x in out.splitlines() if x.startswith("{")]


def test_more_than_one_gpu_is_refused(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_every_workload_has_a_traffic_summary():
    """Each workload names a rocprofv3 FETCH_SIZE/WRITE_SIZE summary under profiles/
    that parses and states a source hash; every config is covered."""
    import os
    import bench_profile
    assert set(bench.TRAFFIC_FILES) == set(synth.CONFIGS)
    for name, rel in bench.TRAFFIC_FILES.items():
        path = os.path.join(bench.ROOT, rel)
        assert os.path.exists(path), rel
        nbytes, digest = bench_profile.read_traffic(path)
        assert nbytes > 0 and len(digest) == 16, rel
        text = open(path).read()
        assert f"--config {name} " in text, rel


def test_algorithmic_bytes():
    p = synth.make_problem("f16", 64, 64, 64, batch=8192, seed=4)
    # A + B (2 bytes) read once, C (fp32) read once, D (fp32) written once
    assert bench.algorithmic_bytes(p) == 8192 * (2 * 4096 * 2 + 2 * 4096 * 4)
    assert bench.algorithmic_bytes(p, "f16", "f16") == 8192 * (2 * 4096 * 2 + 2 * 4096 * 2)
    assert bench.algorithmic_bytes(p, "none", "bf16") == 8192 * (2 * 4096 * 2 + 4096 * 2)
    # 2:4 A: half the values plus four index bits per group of four k
    q = synth.make_problem("bf16", 256, 128, 512, seed=9)
    dense = bench.algorithmic_bytes(q)
    sparse = bench.algorithmic_bytes(q, sparse=True)
    assert dense - sparse == 256 * 512 * 2 - (256 * 512 + 256 * 512 // 8)
    r = synth.make_problem("i8", 256, 128, 512, c_range=(-8, 8), seed=10)
    assert bench.algorithmic_bytes(r, sparse=True) == \
        256 * 512 // 2 + 256 * 512 // 8 + r.B.nbytes + 2 * r.C.nbytes


def test_rotated_workloads_exceed_the_memory_side_cache():
    """The inputs read by the other rotated sets (D bypasses the cache) are at
    least three times the 256 MB memory-side cache."""
    esz = {"f16": 2, "bf16": 2, "i8": 1, "f64": 8}
    csz = {"f16": 4, "bf16": 4, "i8": 4, "f64": 8}
    for name in bench.ROTATE:
        c = synth.CONFIGS[name]
        b = c.get("batch", 1)
        reads = b * (esz[c["dtype"]] * (c["M"] + c["N"]) * c["K"] + csz[c["dtype"]] * c["M"] * c["N"])
        assert (bench.ROTATE_SETS - 1) * reads >= 3 * 256e6, name


def test_cpu_baseline_record():
    p = synth.config_problem("C1")
    rec = bench.cpu_baseline(p, budget_s=0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and 1 <= rec["cores"] <= 16
    assert "of the same seeded problem" in rec["sample"]


def test_single_core_oracle_record():
    rec = bench.single_core_c1()
    assert rec["cores"] == 1 and rec["kind"] == "oracle" and rec["value"] > 0


def check_line(line, metric_unit, config):
    d = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
              "parity"):
        assert k in d, k
    assert d["metric"] == bench.METRIC and d["n_gpus"] == 1 and d["unit"] == metric_unit
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["data"] == "synthetic"
    assert d["config"]["workload"] == synth.CONFIG_LABELS[config]
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and 0 < roof["frac"] < 1
    assert abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-3
    assert d["parity"]["ok"], d["parity"]
    return d


@pytest.mark.gpu
@pytest.mark.parametrize("config,extra,unit", [
    ("C1", [], "TFLOP/s"),
    ("C4", [], "TFLOP/s"),
    ("C3", ["--steps", "3", "--warmup", "1"], "TOP/s"),
    ("SP1", [], "TFLOP/s"),
    ("C2", ["--d-type", "bf16", "--c-type", "none"], "TFLOP/s"),
])
def test_bench_line_on_gpu(capsys, config, extra, unit):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    args = ["--config", config, "--steps", "5", "--warmup", "2", "--no-cpu", *extra]
    with capsys.disabled():
        print(f"[bench] {' '.join(args)}", flush=True)
    lines = run_bench(capsys, *args)
    assert len(lines) == 1, lines
    d = check_line(lines[0], unit, config)
    assert d["config"]["input_sets"] == (bench.ROTATE_SETS if config in bench.ROTATE else 1)
    if config == "C4":
        assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    if config == "SP1":
        assert d["roofline"]["peak"] == bench.SPARSE_PEAK_TFLOPS["bf16"]


@pytest.mark.gpu
def test_bench_study_switches(capsys):
    """--zero-operands labels its line and still checks parity (an exact zero result under a
    zero bound); --settle-ms adds untimed steps and says how many."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with capsys.disabled():
        print("[bench] study switches on the 256^3 fp16 workload", flush=True)
    lines = run_bench(capsys, "--config", "C1", "--steps", "5", "--warmup", "2", "--no-cpu",
                      "--zero-operands", "--settle-ms", "20")
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["data"] == "synthetic, A and B all zeros" and d["config"]["zero_operands"]
    assert d["parity"]["ok"], d["parity"]
    assert d["config"]["settle_ms"] == 20 and d["config"]["settle_steps"] > 0


@pytest.mark.gpu
def test_bench_default_line_with_cpu_baseline(capsys):
    """The driver's invocation (default workload), with the CPU-oracle leg."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with capsys.disabled():
        print("[bench] default workload, 20 steps", flush=True)
    lines = run_bench(capsys, "--steps", "20", "--warmup", "5", "--cpu-budget", "2")
    assert len(lines) == 1, lines
    d = check_line(lines[0], "TFLOP/s", "C2")
    reps = d["config"]["rep_ms_per_step"]
    assert len(reps) == d["config"]["repetitions"] == 5
    assert d["ms_per_step"] == round(sorted(reps)[2], 5)
    # the warm-up is exactly the requested one: no untimed steps beyond it
    assert d["config"]["settle_ms"] == 0 and d["config"]["settle_steps"] == 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["single_core_c1"]["cores"] == 1 and cb["single_core_c1"]["value"] > 0
    # the fp16 and int8 products the metric names, timed in the same run
    other = d["other_dtypes"]
    assert set(other) == set(bench.EXTRA_WORKLOADS)
    for name, unit in (("S1", "TFLOP/s"), ("C3", "TOP/s")):
        o = other[name]
        assert o["workload"] == synth.CONFIG_LABELS[name] and o["unit"] == unit
        assert o["value"] > 0 and o["ms_per_step"] > 0 and len(o["rep_ms_per_step"]) == 5
        assert o["settle_steps"] == 0
        assert o["roofline"]["bound"] == "mfma" and 0 < o["roofline"]["frac"] < 1
        assert o["parity"]["ok"], o["parity"]


@pytest.mark.gpu
def test_smoke_entry_point():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__.smoke()  # raises on a mismatch against the oracle


def test_parity_ratio_of_exact_zero_results():
    """A zero row of A (or all-zero operands) with a zero C gives a zero bound; an exact result
    there counts as error 0, a wrong one as infinitely far outside the bound."""
    import numpy as np
    assert bench._err_over_bound([0.0, 1e-9], [0.0, 1e-6]) == 1e-3
    assert bench._err_over_bound([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert bench._err_over_bound([1e-30], [0.0]) == float("inf")
    p = synth.config_problem("C1")
    p.A[...] = 0
    p.B[...] = 0
    p.C[...] = 0
    D = np.zeros((p.batch, p.M, p.ldc), dtype=np.float32)
    r = bench.parity_sample(p, D)
    assert r["ok"] and r["max_err_over_bound"] == 0.0
    D[...] = 1e-30
    assert not bench.parity_sample(p, D)["ok"]
