"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device, and every workload name it offers
exists in the synthetic workload table."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_bench_workloads_exist():
    import re

    from synth.workloads import ALL

    with open(os.path.join(ROOT, "bench.py")) as f:
        text = f.read()
    m = re.search(r'choices=\[([^\]]*)\]', text)
    names = re.findall(r'"([^"]+)"', m.group(1))
    assert names and all(n in ALL for n in names)
