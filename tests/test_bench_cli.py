"""bench.py's contract on the host (CPU only): it measures one GPU and says so
for any other count, rejects flag combinations it does not time, and counts
the algorithmic bytes of the configurations it reports on."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, env=e, cwd=ROOT)


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_module", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = _run(*args, env=env)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("flags", [["--mx", "--pow2"],
                                   ["--dedup", "--fused"], ["--dedup", "--f16"], ["--mx", "--pow2", "--fp8-combine"],
                                   ["--mn-scales", "--fp8-combine"], ["--mn-convert", "--mn-scales"],
                                   ["--mn-convert", "--dedup"], ["--graph", "--graph-steps", "3"],
                                   ["--graph", "--graph-steps", "0"]])
def test_flag_combinations_it_does_not_time_are_rejected(flags):
    r = _run(*flags)
    assert r.returncode == 2 and r.stdout == "", (flags, r.stderr)


def test_ideal_bytes_of_the_survey_configurations(bench):
    """Config 2 (the metric's), 3 and 5 of the scope table: dispatch and combine
    bytes in MB as tabulated there (x read once, rows written once, y read
    once, out written once, index/weight/scale traffic included)."""
    mb = lambda b: b / 1e6
    d = bench.ideal_bytes(8192, 7168, 256, 8, 8, 65536, fp8=True)
    assert abs(mb(d["dispatch"]) - 601.9) < 0.5 and abs(mb(d["combine"]) - 1057.5) < 0.05
    assert abs(mb(d["dispatch"] + d["combine"]) - 1659.4) < 0.5
    d = bench.ideal_bytes(8192, 7168, 256, 8, 8, 65536, fp8=False)
    assert abs(mb(d["dispatch"]) - 1057.0) < 0.5 and abs(mb(d["combine"]) - 1057.5) < 0.05
    d = bench.ideal_bytes(65536, 4096, 64, 8, 6, 393216, fp8=True)
    assert abs(mb(d["dispatch"]) - 2197.8) < 2.0 and abs(mb(d["combine"]) - 3761.2) < 0.5
    # the layout's own traffic is a fraction of a percent of the step's
    assert d["layout"] < 5e6 and bench.ideal_bytes(8192, 7168, 256, 8, 8, 65536, True)["layout"] < 1e6


def test_ideal_bytes_fp8_combine_and_dedup(bench):
    d = bench.ideal_bytes(8192, 7168, 256, 8, 8, 65536, fp8=True, fp8_combine=True)
    assert abs(d["combine"] / 1e6 - 602.4) < 0.1          # codes + scales instead of bf16 rows
    # dedup with every token reaching all 8 groups moves what the per-expert path does
    full = bench.ideal_bytes_dedup(8192, 7168, 8, 8, 8, 65536, fp8=True)
    per_expert = bench.ideal_bytes(8192, 7168, 256, 8, 8, 65536, fp8=True)
    assert abs(full["dispatch"] - per_expert["dispatch"]) <= 4 * 65536
    fewer = bench.ideal_bytes_dedup(8192, 7168, 8, 8, 8, 43418, fp8=True)
    assert fewer["dispatch"] < full["dispatch"] and fewer["combine"] < full["combine"]
