"""The two-kernel prefill's window plan, checked on the CPU: the host code that
decides which sequences take part in each window and how long it is
(gated_delta_rule_99_amd/csrc/kda_window_plan.h) is compiled with g++ into a
small driver (window_plan_driver.cpp) that checks, for random batches and tile
spaces, that every tile the two kernels can touch lies inside the workspace and
that the windows cover every chunk."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "gated_delta_rule_99_amd", "csrc")


def test_window_plan_bounds(tmp_path):
    exe = os.path.join(tmp_path, "window_plan_driver")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I", CSRC,
                    os.path.join(HERE, "window_plan_driver.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
