"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message (this build has no multi-GPU path), every named workload is
accepted by the parser, and the fraction of peak at the sampled clock scales
with the clock."""
import os
import subprocess
import sys

import tg_inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_workload_is_a_parser_choice():
    r = run("--help")
    assert r.returncode == 0
    text = " ".join(r.stdout.split())
    for name in list(gen.WORKLOADS) + list(gen.ATTN_WORKLOADS):
        assert name in text, name


def test_fraction_of_peak_at_the_sampled_clock():
    sys.path.insert(0, ROOT)
    import bench
    board = {"gfx_clock_mhz_mean": 1200}
    # half the nominal clock: the fraction doubles
    assert bench.at_sampled_clock(board, 0.25 * bench.PEAK_TFLOPS,
                                  bench.PEAK_TFLOPS)["frac_of_peak_at_sampled_clock"] == 0.5
    assert bench.at_sampled_clock(None, 1.0, 2.0) is None
    assert "frac_of_peak_at_sampled_clock" not in bench.at_sampled_clock({}, 1.0, 2.0)
